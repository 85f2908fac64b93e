"""Seeded synthetic inputs for paged decode attention.

This module draws random numbers and places them; it holds none of the
attention or merge arithmetic.  It is the one module that both the GPU path's
callers (tests, bench) and the float64 oracle's callers use, so that both
sides see the same bf16 bits.

Workloads (shapes of the pages' workloads; the data itself is synthetic):
  * tiny      - 1 request, 1 layer, 4,096 tokens, tile 1,024.
  * conc      - 4 requests x 31,744 tokens, 16 layers, tile 8,192: the
                four-request shape on the "Staging without a stall" page.
  * long262k  - 1 request x 262,144 tokens, 16 layers, in eight 32,768-token
                staging tiles: the 262K context on the KV-cache engineering
                page and the 32K staging tiles on the GPU memory management
                page ("Pages held by right, borrowed or free"); 1 % of keys
                scaled by 4 to make the softmax peaked.
  * mixed     - 16 requests, log-uniform lengths in [1,024, 131,072].
  * merge     - 64 x 24 x 256 partials of width 256 for the merge alone.
Head shape for all: 24 query heads, 4 KV heads, head_dim 256, bf16, 64-token
pages, so one token of one layer holds 4 x 256 x 2 x 2 = 4,096 bytes of K+V
(the figure on the GPU memory management page, "A host pool that explains
its own size").

Two generators, same distributions:
  * host   - numpy Philox keyed by (seed, tags); bf16 by round-to-nearest-
             even in integer arithmetic.  Exact and machine independent.
  * device - torch's Philox on the GPU (bf16 by torch's own round-to-nearest-
             even), for full-size workloads whose host generation would take
             minutes.  Regenerating a layer with the same tags gives the same
             bits, which is how the oracle gets its copy.

Pool layout written here (the library header documents the same layout):
  arena = layers[L] x pages[P] x [K | V] x kv heads[Hkv] x one 32 KiB block
  (64 tokens x 256 channels, bf16).  A block is 2,048 pieces of 16 bytes
  (8 bf16) stored in the order the decode kernel's wave loads consume them,
  64 pieces (1 KiB) per load instruction:
    K piece (token j, channels 8c..8c+7) sits at
        ((h*2 + t)*8 + c//4)*64 + (c%4)*16 + r
      with h = j//32, jj = j%32, t = (jj//4)%2, r = 4*(jj//8) + jj%4;
    V piece (channel d, tokens 8u..8u+7) sits at
        ((u//4)*16 + d//16)*64 + (u%4)*16 + d%16.
"""

from dataclasses import dataclass, field
import math

import numpy as np

PAGE_TOKENS = 64
BF16_QNAN = 0x7FC0


# ----------------------------------------------------------------------------
# random streams and bf16 rounding


def rng(seed, *tags):
    """numpy Generator on a Philox stream keyed by (seed, *tags)."""
    ss = np.random.SeedSequence([int(seed)] + [int(t) for t in tags])
    return np.random.Generator(np.random.Philox(ss))


def seed64(seed, *tags):
    """A 63-bit seed derived from (seed, *tags), for torch generators."""
    ss = np.random.SeedSequence([int(seed)] + [int(t) for t in tags])
    return int(ss.generate_state(1, np.uint64)[0] >> np.uint64(1))


def bf16_bits(x):
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even.

    Adds 0x7FFF plus the lowest kept bit to the binary32 word and keeps the
    upper 16 bits.  Inputs must be finite and below bf16's largest finite
    value (true for every draw here).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


# tags that keep the streams of different tensors apart
T_Q, T_K, T_V, T_BOOST, T_TABLE, T_CTX, T_STRESS = 1, 2, 3, 4, 5, 6, 7


# ----------------------------------------------------------------------------
# workloads


@dataclass
class Workload:
    name: str
    seed: int
    ctx_lens: list
    num_layers: int
    tile_tokens: int
    num_q_heads: int = 24
    num_kv_heads: int = 4
    head_dim: int = 256
    page_tokens: int = PAGE_TOKENS
    boost_frac: float = 0.0        # fraction of keys scaled by 4 per (layer, kv head)
    stage_tokens: int = 0          # staging-tile length (0: not staged)
    arena_pages: int = 0           # 0: exactly the pages the requests use
    extra: dict = field(default_factory=dict)

    @property
    def batch(self):
        return len(self.ctx_lens)

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def pages_per_req(self):
        return [-(-c // self.page_tokens) for c in self.ctx_lens]

    @property
    def max_ctx(self):
        return max(self.ctx_lens) if self.ctx_lens else 0

    @property
    def pt_stride(self):
        return max(1, -(-self.max_ctx // self.page_tokens))

    @property
    def num_pages(self):
        return self.arena_pages or sum(self.pages_per_req)

    @property
    def page_layer_bytes(self):
        return 2 * self.num_kv_heads * self.page_tokens * self.head_dim * 2

    @property
    def kv_bytes_per_step(self):
        """K+V bytes the exact path must read per decode step (all layers)."""
        return sum(self.ctx_lens) * self.num_kv_heads * self.head_dim * 2 * 2 * self.num_layers


def mixed_ctx_lens(seed, batch, lo=1024, hi=131072):
    """Log-uniform context lengths: floor(exp(U)), U ~ Uniform(ln lo, ln hi)."""
    u = rng(seed, T_CTX).uniform(math.log(lo), math.log(hi), size=batch)
    return [int(min(max(math.floor(math.exp(x)), lo), hi)) for x in u]


def workload(name, **over):
    """The named workload; keyword arguments override fields (tests use this
    to shrink layer counts)."""
    if name == "tiny":
        w = Workload("tiny", seed=1, ctx_lens=[4096], num_layers=1, tile_tokens=1024)
    elif name == "conc":
        # 8 GiB arena = 2,048 pages of 4 MiB (16 layers x 256 KiB); the four
        # requests take 1,984 of them at random.
        w = Workload("conc", seed=2, ctx_lens=[31744] * 4, num_layers=16,
                     tile_tokens=8192, arena_pages=2048)
    elif name == "long262k":
        w = Workload("long262k", seed=3, ctx_lens=[262144], num_layers=16,
                     tile_tokens=1024, boost_frac=0.01, stage_tokens=32768,
                     arena_pages=4096)
    elif name == "mixed":
        w = Workload("mixed", seed=4, ctx_lens=mixed_ctx_lens(4, 16), num_layers=16,
                     tile_tokens=1024)
    else:
        raise KeyError(name)
    for k, v in over.items():
        setattr(w, k, v)
    return w


# ----------------------------------------------------------------------------
# host (numpy) draws


def draw_q(w, layer):
    """q for every request of one layer: uint16 bf16 bits [B, Hq, D]."""
    x = rng(w.seed, T_Q, layer).standard_normal((w.batch, w.num_q_heads, w.head_dim),
                                                dtype=np.float32)
    return bf16_bits(x)


def boost_positions(w, layer, b, g, ctx):
    """Token positions whose K row is scaled by 4 (exactly round(frac*ctx),
    drawn without replacement per (layer, request, kv head))."""
    n = int(round(w.boost_frac * ctx))
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(rng(w.seed, T_BOOST, layer, b, g).choice(ctx, size=n, replace=False))


def draw_kv(w, layer, b):
    """Logical K and V of one request and layer: uint16 bf16 bits
    [Hkv, ctx, D] each, token order 0..ctx-1.  Each (layer, request, KV head)
    has its own stream, drawn token by token, so a shorter history is a
    prefix of a longer one (boosted positions aside)."""
    ctx = w.ctx_lens[b]
    k = np.empty((w.num_kv_heads, ctx, w.head_dim), dtype=np.float32)
    v = np.empty_like(k)
    for g in range(w.num_kv_heads):
        k[g] = rng(w.seed, T_K, layer, b, g).standard_normal((ctx, w.head_dim), dtype=np.float32)
        v[g] = rng(w.seed, T_V, layer, b, g).standard_normal((ctx, w.head_dim), dtype=np.float32)
        idx = boost_positions(w, layer, b, g, ctx)
        k[g, idx] *= 4.0                      # exact: a power of two
    return bf16_bits(k), bf16_bits(v)


def draw_page_tables(w, width=None):
    """int32 page tables [B, width]: a seeded permutation of the arena's
    pages, request 0 taking the first ceil(ctx_0/64) entries, request 1 the
    next, and so on; unused entries are -1.  Row b's entry 0 is its sink page.
    width defaults to w.pt_stride (the longest request's page count)."""
    P = w.num_pages
    need = sum(w.pages_per_req)
    if need > P:
        raise ValueError(f"workload needs {need} pages, arena has {P}")
    width = w.pt_stride if width is None else width
    if width < w.pt_stride:
        raise ValueError(f"width {width} < {w.pt_stride} pages of the longest request")
    perm = rng(w.seed, T_TABLE).permutation(P).astype(np.int32)
    table = np.full((w.batch, width), -1, dtype=np.int32)
    o = 0
    for b, n in enumerate(w.pages_per_req):
        table[b, :n] = perm[o:o + n]
        o += n
    return table


def _k_piece_order():
    """For each storage position of a K block, the logical piece j*32 + c
    (token j, channels 8c..8c+7) it holds."""
    order = np.empty(2048, dtype=np.int64)
    for j in range(64):
        h, jj = divmod(j, 32)
        t, r = (jj // 4) % 2, 4 * (jj // 8) + jj % 4
        for c in range(32):
            order[((h * 2 + t) * 8 + c // 4) * 64 + (c % 4) * 16 + r] = j * 32 + c
    return order


def _v_piece_order():
    """For each storage position of a V block, the logical piece d*8 + u
    (channel d, tokens 8u..8u+7) it holds."""
    order = np.empty(2048, dtype=np.int64)
    for d in range(256):
        for u in range(8):
            order[((u // 4) * 16 + d // 16) * 64 + (u % 4) * 16 + d % 16] = d * 8 + u
    return order


K_PIECES = _k_piece_order()
V_PIECES = _v_piece_order()


def page_blocks(k_bits, v_bits, page_tokens, pad_value=0):
    """Logical K/V [Hkv, ctx, 256] -> per-page blocks in pool layout,
    [npages, Hkv, 64*256] each.  Tokens past ctx in the last page get
    pad_value (a bf16 bit pattern)."""
    Hkv, ctx, D = k_bits.shape
    assert D == 256 and page_tokens == 64
    n = -(-ctx // page_tokens)
    kp = np.full((Hkv, n * page_tokens, D), pad_value, dtype=np.uint16)
    vp = np.full((Hkv, n * page_tokens, D), pad_value, dtype=np.uint16)
    kp[:, :ctx] = k_bits
    vp[:, :ctx] = v_bits
    kl = kp.reshape(Hkv, n, 64 * 32, 8)                               # pieces j*32 + c
    vl = vp.reshape(Hkv, n, 64, 256).transpose(0, 1, 3, 2).reshape(Hkv, n, 256 * 8, 8)
    kb = kl[:, :, K_PIECES].reshape(Hkv, n, 64 * D).transpose(1, 0, 2)
    vb = vl[:, :, V_PIECES].reshape(Hkv, n, 64 * D).transpose(1, 0, 2)
    return np.ascontiguousarray(kb), np.ascontiguousarray(vb)


def host_pool(w, table, layers=None, fill=0, pad_value=None):
    """Build the whole arena on the host as uint16 [L, P, 2, Hkv, 64*D] and
    return (pool, kv) with kv[(layer, b)] = (k_bits, v_bits) logical.

    layers: which layers to fill (default all); the rest keep `fill`.
    fill: bf16 pattern for every byte no request owns (BF16_QNAN poisons)."""
    if pad_value is None:
        pad_value = fill
    L, Hkv, D, PT = w.num_layers, w.num_kv_heads, w.head_dim, w.page_tokens
    pool = np.full((L, w.num_pages, 2, Hkv, PT * D), fill, dtype=np.uint16)
    kv = {}
    for layer in (range(L) if layers is None else layers):
        for b in range(w.batch):
            kbits, vbits = draw_kv(w, layer, b)
            kv[(layer, b)] = (kbits, vbits)
            n = w.pages_per_req[b]
            if n == 0:
                continue
            kb, vb = page_blocks(kbits, vbits, PT, pad_value)
            pages = table[b, :n]
            pool[layer, pages, 0] = kb
            pool[layer, pages, 1] = vb
    return pool, kv


# ----------------------------------------------------------------------------
# device (torch) draws for full-size workloads


def device_kv(w, layer, b, device):
    """Logical K, V of one request and layer as torch bf16 [Hkv, ctx, D] on
    `device`, from torch's Philox seeded per (seed, layer, request, KV head)."""
    import torch
    ctx = w.ctx_lens[b]
    k = torch.empty((w.num_kv_heads, ctx, w.head_dim), dtype=torch.bfloat16, device=device)
    v = torch.empty_like(k)
    gen = torch.Generator(device=device)
    for g in range(w.num_kv_heads):
        gen.manual_seed(seed64(w.seed, T_K, layer, b, g))
        kf = torch.randn((ctx, w.head_dim), generator=gen, device=device, dtype=torch.float32)
        idx = boost_positions(w, layer, b, g, ctx)
        if len(idx):
            kf[torch.from_numpy(idx).to(device)] *= 4.0
        k[g] = kf.to(torch.bfloat16)
        del kf
        gen.manual_seed(seed64(w.seed, T_V, layer, b, g))
        v[g] = torch.randn((ctx, w.head_dim), generator=gen, device=device,
                           dtype=torch.float32).to(torch.bfloat16)
    return k, v


def device_q(w, layer, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed64(w.seed, T_Q, layer))
    return torch.randn((w.batch, w.num_q_heads, w.head_dim), generator=g, device=device,
                       dtype=torch.float32).to(torch.bfloat16)


def device_scatter(pool, w, layer, b, table_row, k, v, pad_value=0):
    """Write logical K, V (torch bf16 [Hkv, ctx, 256]) of one request into the
    arena `pool` (a contiguous torch int16 tensor of L x P pages, any shape)
    at the pages of `table_row`, in the pool layout."""
    import torch
    Hkv, ctx, D = k.shape
    PT = w.page_tokens
    n = -(-ctx // PT)
    if n == 0:
        return
    dev = pool.device
    pages = torch.as_tensor(np.asarray(table_row[:n], dtype=np.int64), device=dev)
    p5 = pool.view(torch.int16).reshape(-1).view(w.num_layers, -1, 2, Hkv, PT * D)
    pad16 = int(np.uint16(pad_value).view(np.int16))

    def padded(x):
        y = torch.full((Hkv, n * PT, D), pad16, dtype=torch.int16, device=dev)
        y[:, :ctx] = x.view(torch.int16)
        return y
    kp, vp = padded(k), padded(v)
    kl = kp.view(Hkv, n, 64 * 32, 8)
    vl = vp.view(Hkv, n, 64, 256).transpose(2, 3).reshape(Hkv, n, 256 * 8, 8)
    kidx = torch.as_tensor(K_PIECES, device=dev)
    vidx = torch.as_tensor(V_PIECES, device=dev)
    kb = kl[:, :, kidx].reshape(Hkv, n, PT * D).permute(1, 0, 2)
    vb = vl[:, :, vidx].reshape(Hkv, n, PT * D).permute(1, 0, 2)
    p5[layer, pages, 0] = kb.contiguous()
    p5[layer, pages, 1] = vb.contiguous()


# ----------------------------------------------------------------------------
# compact (one byte per element) block layout: where each (token, channel)
# code of a 64 x 256 block sits among the block's 16,384 bytes


def _kc_byte_map():
    """[64 tokens, 256 channels] -> byte offset in a compact K block."""
    out = np.empty((64, 256), dtype=np.int64)
    for ld in range(16):                        # load index (h*2 + t)*4 + kk
        h, t, kk = ld // 8, (ld // 4) % 2, ld % 4
        for lane in range(64):
            q, r = lane // 16, lane % 16
            j = 32 * h + 8 * (r // 4) + 4 * t + r % 4
            piece = ld * 64 + lane
            for e in range(8):
                out[j, 64 * kk + 8 * q + e] = piece * 16 + e
                out[j, 64 * kk + 32 + 8 * q + e] = piece * 16 + 8 + e
    return out


def _vc_byte_map():
    """[64 tokens, 256 channels] -> byte offset in a compact V block."""
    out = np.empty((64, 256), dtype=np.int64)
    for db in range(16):
        for lane in range(64):
            q, d = lane // 16, 16 * db + lane % 16
            piece = db * 64 + lane
            for e in range(8):
                out[8 * q + e, d] = piece * 16 + e
                out[32 + 8 * q + e, d] = piece * 16 + 8 + e
    return out


KC_BYTES = _kc_byte_map()
VC_BYTES = _vc_byte_map()


def compact_block_image(codes, kind):
    """Codes [64, 256] (token, channel) -> the block's 16,384 bytes."""
    m = KC_BYTES if kind == "k" else VC_BYTES
    img = np.zeros(64 * 256, dtype=np.uint8)
    img[m] = codes
    return img


def compact_block_codes(image, kind):
    """The block's 16,384 bytes -> codes [64, 256] (token, channel)."""
    m = KC_BYTES if kind == "k" else VC_BYTES
    return np.asarray(image, dtype=np.uint8)[m]


# ----------------------------------------------------------------------------
# merge stress draws


def stress_draws(seed=5, batch=64, heads=24, tiles=256, keys=4, dim=256,
                 lse_lo=-40.0, lse_hi=40.0, empty_frac=0.1):
    """Random draws for the merge stress test.  Returns a dict with
      r [B,H,T,n] raw key scores ~ N(0,1), vals [B,H,T,n,D] ~ N(0,1),
      target_lse [B,H,T] ~ U[lse_lo, lse_hi], empty bool [B,H,T] ~ Bernoulli,
    with row (0, 0) forced all-empty and row (0, 1) forced to exactly one
    non-empty partial."""
    g = rng(seed, T_STRESS)
    r = g.standard_normal((batch, heads, tiles, keys))
    vals = g.standard_normal((batch, heads, tiles, keys, dim))
    target = g.uniform(lse_lo, lse_hi, size=(batch, heads, tiles))
    empty = g.random((batch, heads, tiles)) < empty_frac
    empty[0, 0, :] = True
    if heads > 1:
        empty[0, 1, :] = True
        empty[0, 1, tiles // 2] = False
    return dict(r=r, vals=vals, target_lse=target, empty=empty)


# ----------------------------------------------------------------------------
# a live-pool schedule: the 4-request shape growing by one token per step in
# a device pool smaller than the histories


def live_schedule(steps=20):
    """Four requests of about 31,744 tokens, each growing by one token per
    step it takes part in (the new token counts in the step's length; a
    paused request keeps its length), served from a device
    pool of 1,491 pages, three quarters of the 1,988 pages the final
    histories fill.  The starting lengths differ by a few tokens, so the
    requests open their 497th page at different steps.  Targets and bursts
    (pages) change mid-run and one request pauses for a step, so that every
    source of a page is used: reuse of an own page, free pages, borrowed,
    above-target and idle reclamation, and shrinking.

    Returns dict(pool_pages, start [4], contexts {id: (target, burst)},
    steps [list of dict(ids, lengths, set_target {id: (target, burst)})],
    final [4]).  Lengths are tokens including the step's new token."""
    start = [31744 - 9, 31744 - 5, 31744 - 13, 31744 - 1]
    contexts = {0: (300, 200), 1: (300, 200), 2: (400, 0), 3: (380, 0)}
    retarget = {8: {2: (300, 0), 0: (600, 0)}, 12: {1: (500, 0)}}
    paused = {12: {3}}
    plan = []
    length = list(start)
    for s in range(1, steps + 1):
        ids = [c for c in range(4) if c not in paused.get(s, set())]
        for c in ids:
            length[c] += 1
        plan.append(dict(ids=ids, lengths=[length[c] for c in ids],
                         set_target=retarget.get(s, {})))
    return dict(pool_pages=1491, start=start, contexts=contexts, steps=plan, final=length)
