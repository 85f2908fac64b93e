"""Float64 reference for decode attention over a paged KV history, tile
partials and their log-sum-exp merge.

TEST INFRASTRUCTURE, NOT PRODUCT CODE (see the package docstring for who may
call it).  Plain numpy in float64; no blocking, fusion or reordering beyond
what each definition below states.

Sources, by page and section:
  * KV-cache engineering page, "Costing the bus before changing anything":
    on the exact path each new token attends the entire history.
  * KV-cache engineering page, "Exact recent pages, compact older pages":
    a tile gives an output already divided by its own softmax sum, plus the
    log-sum-exp of its scores; the FP32 merge weights partial t by
    exp(lse_t - max_t lse_t), adds the weighted outputs, divides by the total
    weight and reports max + log(total); the result is the softmax of the
    whole key set, and plain averaging of the partial outputs is ruled out.
Readings where the pages are silent (each one is listed in the design notes):
  natural logarithm for the log-sum-exp; the softmax scale is inside the
  scores; q head h reads KV head h // (Hq / Hkv); an empty tile is
  (out = 0, lse = -inf); a merge of only empty tiles is (0, -inf); tiles
  start at logical token 0 and are tile_tokens long, the last one ragged.

Parity pinned by tests/test_oracle.py for every function here.
"""

import numpy as np

NEG_INF = float("-inf")


def widen_bf16(bits):
    """bfloat16 bit patterns (uint16) -> float64, exactly.

    A bfloat16 is the upper half of an IEEE binary32, so placing the 16 bits
    in the high half of a 32-bit word gives the binary32 with the same value,
    and binary32 -> binary64 is exact.
    """
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def attend(s, v):
    """Softmax attention of queries over one set of keys, in one pass.

    s: scores [..., n] (already scaled); v: values [n, D] shared by every
    leading index, or [..., n, D].  Returns (out [..., D], lse [...]) with
    out = sum_j softmax(s)_j v_j and lse = log sum_j exp(s_j), evaluated as
    m + log(sum_j exp(s_j - m)) with m = max_j s_j.  Keys with s = -inf take
    no part.  A row with no keys (n == 0 or every s = -inf) gives (0, -inf).
    """
    s = np.asarray(s, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lead = s.shape[:-1]
    D = v.shape[-1]
    if s.shape[-1] == 0:
        return np.zeros(lead + (D,)), np.full(lead, NEG_INF)
    m = s.max(axis=-1)
    live = np.isfinite(m)
    m_safe = np.where(live, m, 0.0)
    e = np.exp(s - m_safe[..., None])            # exp(-inf) = 0 for masked keys
    Z = e.sum(axis=-1)
    if v.ndim == 2:
        num = e @ v
    else:
        num = np.einsum("...n,...nd->...d", e, v)
    Z_safe = np.where(live, Z, 1.0)
    out = np.where(live[..., None], num / Z_safe[..., None], 0.0)
    lse = np.where(live, m_safe + np.log(Z_safe), NEG_INF)
    return out, lse


def tile_bounds(ctx, tile_tokens, num_tiles):
    """Token ranges [start, end) of tiles 0..num_tiles-1 over a history of
    ctx tokens: tile t covers [t*T, min((t+1)*T, ctx)); a tile starting at or
    after ctx is empty (start == end)."""
    out = []
    for t in range(num_tiles):
        a = min(t * tile_tokens, ctx)
        b = min((t + 1) * tile_tokens, ctx)
        out.append((a, b))
    return out


def _group_scores(q, k, scale, num_kv_heads, g, a, b):
    Hq = q.shape[0]
    G = Hq // num_kv_heads
    heads = slice(g * G, (g + 1) * G)
    return (q[heads] @ k[g, a:b].T) * scale, heads


def tile_partials(q, k, v, scale, bounds, num_kv_heads):
    """Per-tile normalised output and log-sum-exp for one request and layer.

    q: [Hq, D]; k, v: [Hkv, n, D] in logical token order; bounds: list of
    (start, end) token ranges, one per tile, in any sizes (empty allowed).
    Returns (o [Hq, T, D], lse [Hq, T]); an empty tile is (0, -inf).
    """
    q = np.asarray(q, dtype=np.float64)
    Hq, D = q.shape
    T = len(bounds)
    o = np.zeros((Hq, T, D))
    lse = np.full((Hq, T), NEG_INF)
    for t, (a, b) in enumerate(bounds):
        if b <= a:
            continue
        for g in range(num_kv_heads):
            s, heads = _group_scores(q, k, scale, num_kv_heads, g, a, b)
            o[heads, t], lse[heads, t] = attend(s, v[g, a:b])
    return o, lse


def merge(o, lse):
    """The log-sum-exp merge of tile partials.

    o: [..., T, D] normalised tile outputs; lse: [..., T].  With
    M = max_t lse_t: if M = -inf every tile is empty and the result is
    (0, -inf).  Otherwise w_t = exp(lse_t - M) (0 for an empty tile),
    W = sum_t w_t, out = sum_t w_t o_t / W and lse = M + log W.
    Only lse = -inf marks an empty tile: a NaN log-sum-exp is not a tile
    the formula can weigh, and IEEE arithmetic of the formula carries it
    to the row's out and lse (NaN), as it does any NaN input.
    """
    o = np.asarray(o, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    M = lse.max(axis=-1)                       # NaN if any lse of the row is NaN
    empty_row = M == NEG_INF
    empty = lse == NEG_INF
    M_safe = np.where(empty_row, 0.0, M)
    w = np.where(empty, 0.0, np.exp(lse - M_safe[..., None]))
    W = w.sum(axis=-1)
    W_safe = np.where(empty_row, 1.0, W)
    contrib = np.where(empty[..., None], 0.0, w[..., None] * o)
    out = contrib.sum(axis=-2) / W_safe[..., None]
    out = np.where(empty_row[..., None], 0.0, out)
    lse_m = np.where(empty_row, NEG_INF, M_safe + np.log(W_safe))
    return out, lse_m


def decode_one_pass(q, k, v, ctx, scale, num_kv_heads):
    """Exact decode attention of one request and layer over its first ctx
    keys, as one softmax per query head.  q: [Hq, D]; k, v: [Hkv, >=ctx, D].
    Returns (out [Hq, D], lse [Hq])."""
    q = np.asarray(q, dtype=np.float64)
    Hq, D = q.shape
    out = np.zeros((Hq, D))
    lse = np.full(Hq, NEG_INF)
    if ctx <= 0:
        return out, lse
    for g in range(num_kv_heads):
        s, heads = _group_scores(q, k, scale, num_kv_heads, g, 0, ctx)
        out[heads], lse[heads] = attend(s, v[g, :ctx])
    return out, lse


def decode_tiled(q, k, v, ctx, scale, num_kv_heads, tile_tokens, num_tiles):
    """Decode attention computed tile by tile then merged.  Returns
    (o [Hq, T, D], lse_t [Hq, T], out [Hq, D], lse [Hq])."""
    bounds = tile_bounds(ctx, tile_tokens, num_tiles)
    o, lse_t = tile_partials(q, k, v, scale, bounds, num_kv_heads)
    out, lse = merge(o, lse_t)
    return o, lse_t, out, lse


def stress_partials(r, vals, target_lse, empty):
    """Partials for the merge stress test, built from explicit keys.

    r: raw key scores [..., T, n]; vals: key values [..., T, n, D];
    target_lse: [..., T]; empty: bool [..., T].  A non-empty partial t gets
    the key scores c_t + r_tj with c_t = target_lse_t - logsumexp_j(r_tj), so
    its log-sum-exp is target_lse_t; its output is the softmax-weighted mean
    of its values.  An empty partial is (0, -inf) and its keys take no part.
    Returns (o [..., T, D], lse [..., T], scores [..., T, n]); scores is -inf
    for every key of an empty partial.
    """
    r = np.asarray(r, dtype=np.float64)
    _, lse_r = attend(r, np.zeros(r.shape + (1,)))
    c = np.asarray(target_lse, dtype=np.float64) - lse_r
    scores = c[..., None] + r
    scores = np.where(np.asarray(empty)[..., None], NEG_INF, scores)
    o, lse = attend(scores, vals)
    return o, lse, scores


def union_attention(scores, vals):
    """Softmax attention over the union of all keys of all partials.

    scores: [..., T, n] (-inf = key absent); vals: [..., T, n, D].
    Returns (out [..., D], lse [...])."""
    scores = np.asarray(scores, dtype=np.float64)
    vals = np.asarray(vals, dtype=np.float64)
    lead = scores.shape[:-2]
    T, n = scores.shape[-2:]
    D = vals.shape[-1]
    return attend(scores.reshape(lead + (T * n,)), vals.reshape(lead + (T * n, D)))
