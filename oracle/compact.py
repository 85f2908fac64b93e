"""Float64 reference for the compact representation of older pages: 8-bit
floating-point (E4M3) codes with one FP32 scale per block, the attention
over dequantised keys and values, and the CRC-32 published with a converted
page.

TEST INFRASTRUCTURE, NOT PRODUCT CODE (see the package docstring for who may
call it).  Plain numpy; no blocking or reordering beyond the definitions.

Sources, by page and section:
  * KV-cache engineering page, "Exact recent pages, compact older pages":
    a request's history is cut into runs of two representations; a page is
    converted only after every layer has written all its tokens, then
    checksummed and published, and served exact before that.
  * KV-cache engineering page, "What the hybrid tier buys": a representation
    is worth the bus bytes per token it saves.
The pages name no compact format.  Readings (each one is listed in the
design notes):
  * format: E4M3 as in the OCP 8-bit floating-point specification: sign,
    4 exponent bits with bias 7, 3 mantissa bits, subnormals, no infinity,
    S.1111.111 is NaN, largest finite 448;
  * one FP32 scale per (layer, page, K|V, KV head) block of 64 tokens x 256
    channels: scale = amax / 448 computed in FP32 (1 if amax = 0), codes =
    E4M3 rounding (to nearest, ties to even, saturating at +-448, sign kept,
    also for a zero result) of the FP32 quotient x / scale; the value a code
    stands for is code_value * scale;
  * CRC-32 is the common reflected CRC (polynomial 0x04C11DB7, initial value
    and final xor 0xFFFFFFFF) of the compact page's bytes: for each layer in
    order, its code blocks as stored, then its scales (FP32, little endian).

Parity pinned by tests/test_oracle_compact.py for every function here.
"""

import zlib

import numpy as np

E4M3_MAX = 448.0


def e4m3_values():
    """The real value of each of the 256 E4M3 codes (NaN for the two NaN
    codes), from the format's definition."""
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            out[code] = np.nan
        elif e == 0:
            out[code] = sign * m * 2.0 ** -9            # subnormal: m/8 * 2^(1-7)
        else:
            out[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


_VALUES = e4m3_values()
_POS = _VALUES[:127]          # codes 0..126: the non-negative finite values, increasing


def e4m3_encode(y):
    """FP32 values -> E4M3 codes: the nearest finite value, ties to the even
    code (mantissa bit 0), magnitudes past 448 saturate to 448; the code's
    sign is the input's sign bit (so -0.0 and negatives that round to zero
    give 0x80).

    Written out on the value table: the codes 0..126 hold the non-negative
    finite values in increasing order, so |y| lies between the first value
    at or above it (hi) and the one before (lo); the nearer of the two wins,
    an equal distance goes to the code whose lowest bit is 0."""
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y.astype(np.float64))                       # exact
    hi = np.clip(np.searchsorted(_POS, a, side="left"), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_hi = _POS[hi] - a
    d_lo = a - _POS[lo]
    take_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    code = np.where(take_lo, lo, hi)
    code = np.where(a >= E4M3_MAX, 126, code)             # saturate at 448
    return (code.astype(np.uint8) | np.where(np.signbit(y), 0x80, 0).astype(np.uint8)).reshape(
        y.shape)


def e4m3_decode(codes):
    """E4M3 codes -> float64 values (exact)."""
    return _VALUES[np.asarray(codes, dtype=np.uint8)]


def block_scale(x):
    """FP32 scale of one block of FP32 (here: widened bf16) values:
    amax / 448 in FP32, or 1 when the block is all zero."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    if amax == 0:
        return np.float32(1.0)
    return np.float32(amax / np.float32(E4M3_MAX))


def quantize_block(x):
    """One block -> (codes uint8, same shape; scale float32)."""
    x = np.asarray(x, dtype=np.float32)
    s = block_scale(x)
    y = (x / s).astype(np.float32)                  # FP32 quotient, correctly rounded
    return e4m3_encode(y), s


def dequantize(codes, scale):
    """Codes and their block scale -> float64 values (exact products)."""
    return e4m3_decode(codes) * np.float64(scale)


def quantize_history(x, page_tokens=64):
    """A history [tokens, D] (float32 values) cut into blocks of page_tokens
    rows, each quantised with its own scale (quantize_block, applied to all
    blocks at once); a trailing partial block is quantised over the rows it
    has.  Returns (codes [tokens, D], scales [n_blocks] float32)."""
    x = np.asarray(x, dtype=np.float32)
    n, D = x.shape
    full = n // page_tokens
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = []
    if full:
        xb = x[:full * page_tokens].reshape(full, page_tokens, D)
        amax = np.max(np.abs(xb), axis=(1, 2)).astype(np.float32)
        s = np.where(amax == 0, np.float32(1.0),
                     (amax / np.float32(E4M3_MAX)).astype(np.float32)).astype(np.float32)
        y = (xb / s[:, None, None]).astype(np.float32)
        codes[:full * page_tokens] = e4m3_encode(y).reshape(full * page_tokens, D)
        scales.extend(s.tolist())
    if n > full * page_tokens:
        c, s1 = quantize_block(x[full * page_tokens:])
        codes[full * page_tokens:] = c
        scales.append(s1)
    return codes, np.array(scales, dtype=np.float32)


def dequantize_history(codes, scales, page_tokens=64):
    """Inverse of quantize_history's representation: float64 [tokens, D],
    each element value(code) times its block's scale."""
    codes = np.asarray(codes, dtype=np.uint8)
    block = np.arange(codes.shape[0]) // page_tokens
    return e4m3_decode(codes) * np.asarray(scales, dtype=np.float64)[block][:, None]


def crc32(data):
    """CRC-32 (reflected 0x04C11DB7, init and final xor 0xFFFFFFFF) of a byte
    string, by the library routine that computes exactly this definition."""
    return zlib.crc32(bytes(data)) & 0xFFFFFFFF


def lse_error_bound(q, k, k_hat, scale):
    """Upper bound on |lse(q . k_hat) - lse(q . k)| for a query over one set
    of keys: log-sum-exp moves by at most the largest change of any one
    score, and score j changes by scale * |q . (k_hat_j - k_j)|.

    q [D] or [H, D] (several queries over the same keys), k and k_hat
    [n, D] (float64).  Returns a float, or an array [H]."""
    q = np.asarray(q, dtype=np.float64)
    dk = np.asarray(k_hat, dtype=np.float64) - np.asarray(k, dtype=np.float64)
    if dk.shape[0] == 0:
        return 0.0 if q.ndim == 1 else np.zeros(q.shape[0])
    d = np.abs(dk @ q.T)                               # [n] or [n, H]
    return (float(np.max(d)) if q.ndim == 1 else np.max(d, axis=0)) * abs(scale)


def two_runs(x_bits, compact_tokens, page_tokens=64):
    """The values attention sees when a history [tokens, D] of bf16 bit
    patterns is served in two runs: its first compact_tokens tokens (whole
    pages) from compact pages, the rest exact.  float64 [tokens, D]."""
    from .attention import widen_bf16
    if compact_tokens % page_tokens:
        raise ValueError("the compact run covers whole pages")
    x = widen_bf16(x_bits)
    out = x.copy()
    c = min(compact_tokens, x.shape[0])
    if c:
        codes, scales = quantize_history(x[:c].astype(np.float32), page_tokens)
        out[:c] = dequantize_history(codes, scales, page_tokens)
    return out
