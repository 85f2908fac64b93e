"""Compact older pages on the GPU (pkv_compact_convert, pkv_compact_crc and
decode over a compact pool): the conversion writes exactly the oracle's
E4M3 codes and FP32 scales and the CRC-32 of the page's bytes; a history
served as a compact older run plus an exact recent run, each run decoded
with its own table into disjoint slots and merged once, matches the oracle
over the same two-run history; the change from the exact result stays
within the log-sum-exp bound the codes allow.  (KV-cache engineering,
section "Exact recent pages, compact older pages".)"""

import zlib

import numpy as np
import pytest
import torch

from paged_kv_cache_10_amd import inputs as I
from paged_kv_cache_10_amd import pkv
from gpu_helpers import DEV, Case, Runs, assert_lse_close, assert_out_close, same_bits
import oracle
from oracle import compact as C

pytestmark = pytest.mark.gpu

def expected_page(runs, b, i, layer_bits):
    """Oracle codes, scales and CRC-32 of request b's logical page i.
    layer_bits[layer] = (k_bits, v_bits) of the request."""
    w = runs.w
    img = bytearray()
    codes, scales = {}, {}
    for layer in range(w.num_layers):
        kb, vb = layer_bits[layer]
        sc = []
        for kind, bits in (("k", kb), ("v", vb)):
            for g in range(w.num_kv_heads):
                x = oracle.widen_bf16(bits[g, 64 * i:64 * i + 64]).astype(np.float32)
                c, s = C.quantize_block(x)
                codes[(layer, kind, g)] = c
                scales[(layer, kind, g)] = s
                img += I.compact_block_image(c, kind).tobytes()
                sc.append(s)
        img += np.array(sc, dtype="<f4").tobytes()
    return codes, scales, C.crc32(img)


def test_conversion_writes_the_oracle_codes_scales_and_crc(gpu):
    w = I.Workload("cconv", seed=61, ctx_lens=[1000, 4096, 200, 64], num_layers=2,
                   tile_tokens=1024, arena_pages=120)
    case = Case(w)
    runs = Runs(case, [c // 64 * 64 for c in w.ctx_lens])
    codes, scales = runs.compact_bytes()
    crc = runs.crc.cpu().numpy().view(np.uint32)
    bits = {b: {layer: I.draw_kv(w, layer, b) for layer in range(w.num_layers)}
            for b in range(w.batch)}
    k = 0
    for b in range(w.batch):
        for i in range(int(runs.c[b]) // 64):
            dp = runs.ctable[b, i]
            ec, es, ecrc = expected_page(runs, b, i, bits[b])
            for layer in range(w.num_layers):
                for kv, kind in enumerate("kv"):
                    for g in range(w.num_kv_heads):
                        got = I.compact_block_codes(codes[layer, dp, kv, g], kind)
                        np.testing.assert_array_equal(got, ec[(layer, kind, g)],
                                                      err_msg=f"b={b} page={i} {kind}{g} l={layer}")
                        assert scales[layer, dp, kv, g].view(np.uint32) == \
                            np.float32(es[(layer, kind, g)]).view(np.uint32)
            assert crc[k] == ecrc, (b, i, hex(crc[k]), hex(ecrc))
            # the CRC of the bytes as they sit in the arena, by the library routine
            img = b"".join(codes[layer, dp].tobytes() + scales[layer, dp].astype("<f4").tobytes()
                           for layer in range(w.num_layers))
            assert crc[k] == (zlib.crc32(img) & 0xFFFFFFFF)
            k += 1
    # pkv_compact_crc recomputes the published CRCs; an id outside the pool gets 0
    pages = torch.from_numpy(np.append(runs.dst, [-1, 10 ** 6]).astype(np.int32)).to(DEV)
    again = torch.full((pages.numel(),), 7, dtype=torch.int32, device=DEV)
    pkv.compact_crc(runs.pool, pages, again)
    torch.cuda.synchronize()
    again = again.cpu().numpy().view(np.uint32)
    np.testing.assert_array_equal(again[:k], crc[:k])
    assert again[k] == 0 and again[k + 1] == 0


def crafted_case():
    """One 64-token request whose blocks exercise the codes: head 0 cycles
    through every finite E4M3 value, head 1 holds exact midpoints (ties),
    head 2 is all zeros with some -0.0, head 3 is random with one outlier.
    Values are E4M3 values times 2^-6 with +-7 = 448 * 2^-6 present, so the
    scale is 2^-6 and the quotients are the values themselves."""
    w = I.Workload("ccraft", seed=62, ctx_lens=[64], num_layers=1, tile_tokens=64, arena_pages=4)
    case = Case(w)
    vals = C.e4m3_values()
    finite = vals[np.isfinite(vals)]
    mids = (vals[:126] + vals[1:127]) / 2
    r = np.random.default_rng(5)
    blocks = []
    for kind in range(2):
        hs = []
        a = np.resize(r.permutation(finite), 64 * 256)
        a[0] = 448.0
        hs.append(a)
        m = np.resize(np.concatenate([mids, -mids]), 64 * 256)
        m[1] = -448.0
        hs.append(m)
        z = np.zeros(64 * 256)
        z[::7] = -0.0
        hs.append(z)
        x = r.standard_normal(64 * 256) * 0.2
        x[100] = 300.0 if kind == 0 else -250.0
        hs.append(x)
        blocks.append(np.stack(hs).reshape(4, 64, 256) * 2.0 ** -6)
    bits = []
    for blk in blocks:
        b32 = blk.astype(np.float32)
        bits.append(I.bf16_bits(b32))
    k = torch.from_numpy(bits[0].view(np.int16)).view(torch.bfloat16).to(DEV)
    v = torch.from_numpy(bits[1].view(np.int16)).view(torch.bfloat16).to(DEV)
    I.device_scatter(case.arena, w, 0, 0, case.table[0], k, v)
    torch.cuda.synchronize()
    return case, bits


def test_crafted_blocks_cover_every_code_and_tie(gpu):
    case, (kb, vb) = crafted_case()
    w = case.w
    runs = Runs(case, [64])
    codes, scales = runs.compact_bytes()
    dp = runs.ctable[0, 0]
    for kv, (kind, bits) in enumerate((("k", kb), ("v", vb))):
        for g in range(4):
            x = oracle.widen_bf16(bits[g]).astype(np.float32)
            ec, es = C.quantize_block(x)
            np.testing.assert_array_equal(I.compact_block_codes(codes[0, dp, kv, g], kind), ec)
            assert np.float32(scales[0, dp, kv, g]) == es
    seen = set(np.unique(codes[0, dp, :, 0]).tolist())
    assert seen == set(range(256)) - {0x7F, 0xFF}                 # every finite code
    assert np.float32(scales[0, dp, 0, 0]) == np.float32(2.0 ** -6)
    # decode over the crafted page: the whole history is the compact run
    qf = case.q_f64(0)
    got = runs.decode(0, 64)
    k2 = np.stack([C.two_runs(kb[g], 64) for g in range(4)])
    v2 = np.stack([C.two_runs(vb[g], 64) for g in range(4)])
    out, lse = oracle.decode_one_pass(qf[0], k2, v2, 64, w.scale, 4)
    assert_out_close(got[2].cpu().numpy()[0], out)
    assert_lse_close(got[3].cpu().numpy()[0], lse)


RAGGED = [5000, 12345, 64, 700, 33000, 1]


@pytest.mark.parametrize("boundary", ["all_full_pages", "half", "none"])
@pytest.mark.parametrize("tile,split", [(1024, 1024), (4096, 2048)])
def test_two_run_decode_matches_oracle(gpu, boundary, tile, split):
    w = I.Workload("ctwo", seed=63, ctx_lens=RAGGED, num_layers=2, tile_tokens=tile,
                   arena_pages=900)
    case = Case(w)
    if boundary == "all_full_pages":
        c = [n // 64 * 64 for n in w.ctx_lens]
    elif boundary == "half":
        c = [n // 128 * 64 for n in w.ctx_lens]
    else:
        c = [0] * w.batch
    runs = Runs(case, c, seed=len(boundary))
    for layer in range(2):
        got = runs.decode(layer, tile, split)
        runs.check(got, runs.oracle(layer, tile))


def test_two_runs_with_their_own_tilings(gpu):
    """The compact run tiled 3,584 / 3,584 and the exact tail 512 / 512 (the
    262K launch shapes), on ragged lengths."""
    w = I.Workload("ctile", seed=65, ctx_lens=[40000, 7777, 33000], num_layers=1,
                   tile_tokens=512, arena_pages=1300)
    case = Case(w)
    runs = Runs(case, [max(0, (n - 32768) // 64 * 64) for n in w.ctx_lens])
    got = runs.decode(0, 3584, 3584, 512, 512)
    runs.check(got, runs.oracle(0, 3584, etile=512))


@pytest.mark.parametrize("boundary", ["all_full_pages", "half", "none"])
@pytest.mark.parametrize("tile,etile", [(1024, 1024), (4096, 512)])
def test_two_runs_in_one_launch_equal_two_calls_bitwise(gpu, boundary, tile, etile):
    """pkv_decode_attention_runs writes the bits of the two separate calls
    (and so matches the oracle as they do)."""
    w = I.Workload("cone", seed=67, ctx_lens=RAGGED, num_layers=1, tile_tokens=tile,
                   arena_pages=900)
    case = Case(w, fill=I.BF16_QNAN)
    if boundary == "all_full_pages":
        c = [n // 64 * 64 for n in w.ctx_lens]
    elif boundary == "half":
        c = [n // 128 * 64 for n in w.ctx_lens]
    else:
        c = [0] * w.batch
    runs = Runs(case, c, seed=len(boundary))
    sep = runs.decode(0, tile, tile, etile, etile)
    one = runs.decode(0, tile, tile, etile, etile, one_launch=True)
    for x, y in zip(sep, one):
        assert same_bits(x, y)
    runs.check(one, runs.oracle(0, tile, etile=etile))


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 4), (12, 4), (16, 4), (20, 4), (28, 4), (32, 4),
                                    (48, 4), (64, 4), (16, 2)])
def test_compact_query_group_sizes(gpu, hq, hkv):
    """The compact kernel for query groups of 1, 2, 3, 4, 5, 7, 8, 12 and 16 heads per
    KV head, lengths around page edges (every full page compact, the partial
    last page exact), poisoned exact padding."""
    w = I.Workload("cgroups", seed=66, ctx_lens=[130, 2049, 777], num_layers=1,
                   tile_tokens=1024, num_q_heads=hq, num_kv_heads=hkv)
    case = Case(w, fill=I.BF16_QNAN)
    runs = Runs(case, [n // 64 * 64 for n in w.ctx_lens])
    for split in (0, 256):
        got = runs.decode(0, 1024, split)
        runs.check(got, runs.oracle(0, 1024))


def test_compact_decode_is_deterministic_and_agrees_across_splits(gpu):
    w = I.Workload("cdet", seed=64, ctx_lens=[20000, 9000], num_layers=1, tile_tokens=4096,
                   arena_pages=500)
    case = Case(w)
    runs = Runs(case, [16384, 8960])
    a = runs.decode(0, 4096, 4096)
    b = runs.decode(0, 4096, 4096)
    for x, y in zip(a, b):
        assert same_bits(x, y)
    c = runs.decode(0, 4096, 1024)          # another split: same math, other rounding order
    assert_out_close(c[2].cpu().numpy(), a[2].cpu().numpy().astype(np.float64), tol=1e-5)


# ----------------------------------------------------------------------------
# full size: 262,144 tokens, everything but the newest 32,768 tokens compact


@pytest.fixture(scope="module")
def long_runs():
    w = I.workload("long262k")
    case = Case(w, host=False)
    from bench import COMPACT_LAUNCH
    runs = Runs(case, [w.ctx_lens[0] - COMPACT_LAUNCH["long262k"]["exact_tail"]])
    yield runs
    del runs, case
    torch.cuda.empty_cache()


@pytest.mark.parametrize("layer", [0, 15])
def test_long262k_two_runs_match_oracle(gpu, long_runs, layer):
    from bench import COMPACT_LAUNCH
    cl = COMPACT_LAUNCH["long262k"]
    got = long_runs.decode(layer, cl["tile"], cl["split"], cl["exact_tile"], cl["exact_split"],
                           tail_stream=cl["schedule"] == "tail_stream",
                           one_launch=cl["schedule"] == "one_launch")
    long_runs.check(got, long_runs.oracle(layer, cl["tile"], with_exact=False,
                                          etile=cl["exact_tile"]))
    # the runs write disjoint slots: decoding them one after the other on one
    # stream, in two calls, gives the same bits
    serial = long_runs.decode(layer, cl["tile"], cl["split"], cl["exact_tile"], cl["exact_split"])
    for a, b in zip(got, serial):
        assert torch.equal(a, b)


def test_runs_of_one_representation_in_one_launch(gpu):
    """pkv_decode_attention_runs with two exact runs (the history cut at a
    page boundary, each run with its own table) and with one run: the bits
    of the separate pkv_decode_attention calls."""
    w = I.Workload("xruns", seed=68, ctx_lens=[9000, 1500, 0, 4097], num_layers=1,
                   tile_tokens=1024)
    case = Case(w, fill=I.BF16_QNAN)
    B, Hq, D = w.batch, w.num_q_heads, w.head_dim
    cut = 4096                                     # run 0: tokens [0, 4096), run 1: the rest
    c0 = np.minimum(case.ctx, cut).astype(np.int32)
    c1 = np.maximum(case.ctx - cut, 0).astype(np.int32)
    t0 = case.table.copy()
    t0[:, cut // 64:] = -1                         # padding past a run's pages is -1
    t1 = np.full_like(case.table, -1)
    t1[:, :case.table.shape[1] - cut // 64] = case.table[:, cut // 64:]
    t1[c1 == 0] = -1
    dev = {}
    for name, tab, ln in (("r0", t0, c0), ("r1", t1, c1)):
        dt = torch.empty(tab.shape, dtype=torch.int32, device=DEV)
        dc = torch.empty(B, dtype=torch.int32, device=DEV)
        pkv.page_table_write(case.pool, tab, ln, dt, dc)
        dev[name] = (dt, dc)
    S0, S1 = cut // 1024, -(-int(c1.max()) // 512)
    q = case.q[0]

    def fresh():
        return (torch.full((B, Hq, S0 + S1, D), float("nan"), device=DEV),
                torch.full((B, Hq, S0 + S1), float("nan"), device=DEV))
    po, pl = fresh()
    pkv.decode_attention(case.pool, 0, q, dev["r0"][0], dev["r0"][1], 0, S0 * 1024, 1024, w.scale,
                         po, pl, split_tokens=1024)
    pkv.decode_attention(case.pool, 0, q, dev["r1"][0], dev["r1"][1], 0, S1 * 512, 512, w.scale,
                         po, pl, split_tokens=512, slot_offset=S0)
    po2, pl2 = fresh()
    pkv.decode_attention_runs(0, q, [(case.pool, dev["r0"][0], dev["r0"][1], S0 * 1024, 1024, 0),
                                     (case.pool, dev["r1"][0], dev["r1"][1], S1 * 512, 512, S0)],
                              w.scale, po2, pl2)
    torch.cuda.synchronize()
    assert same_bits(po, po2) and same_bits(pl, pl2)
    # the merged result is the softmax over the whole history
    o = torch.empty((B, Hq, D), device=DEV)
    l = torch.empty((B, Hq), device=DEV)
    pkv.merge_partials(po2, pl2, o, l)
    ref = case.oracle_layer(0)
    for b in range(B):
        assert_out_close(o[b].cpu().numpy(), ref[b][2])
        assert_lse_close(l[b].cpu().numpy(), ref[b][3])
    # one run alone: the bits of its own call
    po3, pl3 = fresh()
    pkv.decode_attention_runs(0, q, [(case.pool, dev["r0"][0], dev["r0"][1], S0 * 1024, 1024, 0)],
                              w.scale, po3, pl3)
    torch.cuda.synchronize()
    assert same_bits(po3[:, :, :S0], po[:, :, :S0]) and same_bits(pl3[:, :, :S0], pl[:, :, :S0])


def test_background_conversion_then_publish(gpu):
    """The pages' lifecycle: conversion and CRC run on their own stream while
    exact decode steps go on (their bits unchanged); once the CRC checks,
    the tables switch to the compact run (publish) and the two-run decode
    matches the oracle on the dequantised history."""
    w = I.Workload("cbg", seed=69, ctx_lens=[20000, 9000, 4100], num_layers=2, tile_tokens=2048,
                   arena_pages=600)
    case = Case(w, fill=I.BF16_QNAN)
    ref = [case.decode(layer, tile=2048, split=2048) for layer in range(2)]
    side = torch.cuda.Stream()                     # default priority
    runs = Runs(case, [n // 2048 * 2048 for n in w.ctx_lens], stream=side)
    for _ in range(3):                             # decode steps beside the conversion
        for layer in range(2):
            got = case.decode(layer, tile=2048, split=2048)
            for x, y in zip(got, ref[layer]):
                assert same_bits(x, y)
    side.synchronize()
    total = runs.src.size
    again = torch.empty(total, dtype=torch.int32, device=DEV)
    pkv.compact_crc(runs.pool, runs.dst_dev, again)
    torch.cuda.synchronize()
    assert torch.equal(again, runs.crc[:total])     # the published pages are the converted ones
    for layer in range(2):
        got = runs.decode(layer, 2048, 2048, 1024, 1024, one_launch=True)
        runs.check(got, runs.oracle(layer, 2048, etile=1024))
