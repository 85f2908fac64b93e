"""Pins for the compact-page oracle (CPU only): E4M3 codes, block scales,
dequantisation, CRC-32 and the log-sum-exp error bound, each checked
against something other than itself — the hand-derived fixture
tests/golden/e4m3_codes.json, brute force over the format's value table,
torch's float8_e4m3fn decoding, exact algebraic properties of the format and
of CRC-32's catalogued constants —
and planted mistakes that must each fail a pin."""

import json
import math
import os
import types

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import compact as C

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def num(x):
    x = x.strip()
    if x == "nan":
        return math.nan
    if x == "-0":
        return -0.0
    sign = -1.0 if x.startswith("-") else 1.0
    x = x.lstrip("-")
    if "*" in x:
        a, b = x.split("*")
        return sign * float(a) * num(b)
    if x.startswith("2^"):
        return sign * 2.0 ** int(x[2:])
    return sign * float(x)


def golden():
    with open(os.path.join(GOLDEN, "e4m3_codes.json")) as f:
        return json.load(f)


# ----------------------------------------------------------------------------
# the oracle and planted mutants


def _real():
    return types.SimpleNamespace(encode=C.e4m3_encode, decode=C.e4m3_decode,
                                 quantize=C.quantize_block, crc=C.crc32)


def _mutant(name):
    m = _real()
    if name == "ties_away":                 # ties rounded away from zero
        def enc(y):
            # nudge every magnitude up by one float32 step: ties go away from 0
            y = np.asarray(y, dtype=np.float32)
            return C.e4m3_encode(np.nextafter(np.abs(y), np.float32(np.inf)) * np.where(
                np.signbit(y), np.float32(-1), np.float32(1)))
        m.encode = enc
    elif name == "fnuz_bias":               # exponent bias 8 (another 8-bit format)
        m.decode = lambda c: C.e4m3_decode(c) / 2.0
    elif name == "no_saturate":             # overflow to NaN instead of 448
        def enc(y):
            c = C.e4m3_encode(y)
            big = np.abs(np.asarray(y, dtype=np.float64)) > 448
            return np.where(big, c | 0x7F, c).astype(np.uint8)
        m.encode = enc
    elif name == "scale_240":               # the other format's largest value
        def q(x):
            x = np.asarray(x, dtype=np.float32)
            s = np.float32(np.max(np.abs(x)) / np.float32(240))
            return C.e4m3_encode((x / s).astype(np.float32)), s
        m.quantize = q
    elif name == "truncate":                # rounding toward zero
        def enc(y):
            y = np.asarray(y, dtype=np.float32)
            a = np.abs(y.astype(np.float64))
            idx = np.clip(np.searchsorted(C._POS, a, side="right") - 1, 0, 126)
            return (idx.astype(np.uint8) | np.where(np.signbit(y), 0x80, 0).astype(np.uint8))
        m.encode = enc
    elif name == "crc_no_final_xor":
        m.crc = lambda b: C.crc32(b) ^ 0xFFFFFFFF
    elif name == "unsigned_zero":           # sign dropped when the result is zero
        def enc(y):
            c = C.e4m3_encode(y)
            return np.where((c & 0x7F) == 0, 0, c).astype(np.uint8)
        m.encode = enc
    return m


MUTANTS = ["ties_away", "fnuz_bias", "no_saturate", "scale_240", "truncate", "crc_no_final_xor",
           "unsigned_zero"]


# ----------------------------------------------------------------------------
# pins, each a function of an implementation; the real oracle passes all,
# each mutant fails at least one


def pin_golden_decode(m):
    for code, val in golden()["decode"]:
        got = float(m.decode(np.uint8(int(code, 16))))
        want = num(val)
        if math.isnan(want):
            assert math.isnan(got), code
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), code


def pin_golden_encode(m):
    for val, code in golden()["encode"]:
        got = int(m.encode(np.float32(num(val))))
        assert got == int(code, 16), (val, hex(got), code)


def pin_golden_block(m):
    g = golden()["block"]
    codes, s = m.quantize(np.array(g["x"], dtype=np.float32))
    assert int(np.float32(s).view(np.uint32)) == int(g["scale_bits"], 16)
    assert [[int(c) for c in r] for r in codes] == [[int(c, 16) for c in r] for r in g["codes"]]


def pin_torch_decode(m):
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(m.decode(codes), ref)


def pin_torch_encode(m):
    """torch's float8_e4m3fn conversion rounds to nearest, ties to even; after
    a clamp to +-448 (exact, keeps the sign of zero) it is the encoding."""
    r = np.random.default_rng(11)
    y = np.concatenate([r.standard_normal(20000) * 10.0 ** r.uniform(-5, 3, 20000),
                        (C._POS[:-1] + C._POS[1:]) / 2.0, [0.0, -0.0, 448.0, -500.0]])
    y = y.astype(np.float32)
    t = torch.from_numpy(y).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    np.testing.assert_array_equal(m.encode(y), t.view(torch.uint8).numpy())


def brute_encode(y):
    """The definition by brute force over the value table: the nearest of
    the 127 non-negative finite values to |y| (ties to the even code), past
    448 the largest, with y's sign bit."""
    y = np.asarray(y, dtype=np.float32).ravel()
    vals = C.e4m3_values()[:127]
    out = np.empty(y.size, dtype=np.uint8)
    for i, v in enumerate(y.astype(np.float64)):
        a = abs(v)
        d = np.abs(vals - a)
        best = np.flatnonzero(d == d.min())
        c = int(best[0]) if best.size == 1 else int(best[best % 2 == 0][0])
        out[i] = c | (0x80 if np.signbit(v) else 0)
    return out


def pin_brute_force_encode(m):
    r = np.random.default_rng(7)
    y = np.concatenate([
        r.standard_normal(3000) * 10.0 ** r.uniform(-4, 3, 3000),
        # exact midpoints between neighbouring finite values (all ties)
        (C._POS[:-1] + C._POS[1:]) / 2.0,
        -(C._POS[:-1] + C._POS[1:]) / 2.0,
        [0.0, -0.0, 448.0, 464.0, 470.0, -1e9, 2.0 ** -10, -(2.0 ** -10)],
    ]).astype(np.float32)
    np.testing.assert_array_equal(m.encode(y), brute_encode(y))


def pin_saturation(m):
    y = np.array([448.0, 463.9, 464.0, 500.0, 1e30, -1e30], dtype=np.float32)
    np.testing.assert_array_equal(m.encode(y), [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE])


def pin_round_trip(m):
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = m.decode(codes).astype(np.float32)
    np.testing.assert_array_equal(m.encode(vals), codes)


def pin_block_properties(m):
    """A nonzero block's largest magnitude maps to +-448 exactly; every other
    element is within half a code step (relative 2^-4 in the normal range,
    2^-10 * scale below it); doubling a block doubles its scale and keeps its
    codes; an all-zero block has scale 1 and codes 0."""
    r = np.random.default_rng(11)
    for trial in range(20):
        x = (r.standard_normal((64, 256)) * 10.0 ** r.uniform(-3, 3)).astype(np.float32)
        codes, s = m.quantize(x)
        v = m.decode(codes)
        assert np.max(np.abs(v)) == 448.0
        deq = v * np.float64(s)
        err = np.abs(deq - x.astype(np.float64))
        bound = np.maximum(2.0 ** -4 * np.abs(x.astype(np.float64)), 2.0 ** -10 * float(s)) * (1 + 1e-6)
        assert np.all(err <= bound)
        c2, s2 = m.quantize(x * np.float32(2))
        assert np.float32(s2) == np.float32(2) * np.float32(s)
        np.testing.assert_array_equal(c2, codes)
    codes, s = m.quantize(np.zeros((64, 256), np.float32))
    assert np.float32(s) == 1.0 and not codes.any()


def pin_crc(m):
    g = golden()["crc32"]
    assert m.crc(b"123456789") == int(g["check"], 16)
    r = np.random.default_rng(3)
    for n in (0, 1, 7, 64, 4096):
        msg = r.integers(0, 256, n, dtype=np.uint8).tobytes()
        c = m.crc(msg)
        assert m.crc(msg + c.to_bytes(4, "little")) == int(g["residue"], 16)


PINS = [pin_golden_decode, pin_golden_encode, pin_golden_block, pin_torch_decode,
        pin_torch_encode, pin_brute_force_encode, pin_saturation, pin_round_trip, pin_block_properties, pin_crc]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_passes(pin):
    pin(_real())


@pytest.mark.parametrize("name", MUTANTS)
def test_mutant_is_caught(name):
    m = _mutant(name)
    failed = []
    for pin in PINS:
        try:
            pin(m)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"


# ----------------------------------------------------------------------------
# history helpers and the error bound


def test_history_blocks_have_their_own_scales():
    r = np.random.default_rng(5)
    x = r.standard_normal((150, 256)).astype(np.float32)
    x[64:128] *= 100                                    # second block much larger
    codes, scales = C.quantize_history(x)
    assert scales.shape == (3,)
    for i, b0 in enumerate((0, 64, 128)):
        c, s = C.quantize_block(x[b0:b0 + 64])
        assert s == scales[i]
        np.testing.assert_array_equal(codes[b0:b0 + 64], c)
    deq = C.dequantize_history(codes, scales)
    np.testing.assert_array_equal(deq[64:128], C.dequantize(codes[64:128], scales[1]))


def test_lse_bound_holds_and_is_tight_for_one_key():
    r = np.random.default_rng(9)
    scale = 1 / 16
    for n in (1, 5, 300):
        q = r.standard_normal(256)
        k = r.standard_normal((n, 256)).astype(np.float32)
        codes, scales = C.quantize_history(k)
        k_hat = C.dequantize_history(codes, scales)
        v = r.standard_normal((n, 256))
        _, lse = A.attend(scale * (k.astype(np.float64) @ q), v)
        _, lse_hat = A.attend(scale * (k_hat @ q), v)
        b = C.lse_error_bound(q, k, k_hat, scale)
        assert abs(lse_hat - lse) <= b * (1 + 1e-9) + 1e-15
        if n == 1:
            assert abs(abs(lse_hat - lse) - b) <= 1e-12 * max(1.0, b)
        # several queries at once give each query's own bound
        qs = r.standard_normal((3, 256))
        many = C.lse_error_bound(qs, k, k_hat, scale)
        assert many.shape == (3,)
        for i in range(3):
            assert abs(many[i] - C.lse_error_bound(qs[i], k, k_hat, scale)) <= 1e-12


def test_two_runs_splits_at_the_boundary():
    r = np.random.default_rng(13)
    bits = (r.standard_normal((300, 256)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    x = A.widen_bf16(bits)
    np.testing.assert_array_equal(C.two_runs(bits, 0), x)            # all exact
    got = C.two_runs(bits, 128)
    np.testing.assert_array_equal(got[128:], x[128:])                # exact run untouched
    for b0 in (0, 64):                                               # compact run = pages
        c, s = C.quantize_block(x[b0:b0 + 64].astype(np.float32))
        np.testing.assert_array_equal(got[b0:b0 + 64], C.dequantize(c, s))
    assert not np.array_equal(got[:128], x[:128])
    with pytest.raises(ValueError):
        C.two_runs(bits, 100)


def test_block_scale_definition():
    """block_scale: 1 for an all-zero block, else amax / 448 rounded once to
    FP32 (amax of the magnitudes, the sign of the extreme value ignored)."""
    assert C.block_scale(np.zeros((64, 256), np.float32)) == np.float32(1.0)
    assert C.block_scale(np.array([[0.0, -448.0], [3.0, 1.0]], np.float32)) == np.float32(1.0)
    s = C.block_scale(np.array([[-0.5, 0.25], [1.0, -2.0]], np.float32))
    assert s.dtype == np.float32 and s == np.float32(2.0 / 448.0)
    # 1 / 448 is not a binary fraction: the FP32 rounding of the exact quotient
    exact = 1.0 / 448.0
    s1 = C.block_scale(np.array([1.0], np.float32))
    assert abs(float(s1) - exact) <= abs(float(np.nextafter(s1, np.float32(1))) - float(s1)) / 2
