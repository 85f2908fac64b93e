"""GPU parity: the HIP path (through the C ABI) against the float64 oracle,
element by element, plus the bitwise properties the pages ask of it.

Tolerances: max abs error 2e-3 on outputs and 1e-4 on log-sum-exp."""

import math

import numpy as np
import pytest
import torch

from paged_kv_cache_10_amd import inputs as I
import oracle
from gpu_helpers import (Case, DEV, assert_lse_close, assert_out_close, check_layer, same_bits)

pytestmark = pytest.mark.gpu

KERNELS = ["valu", "mfma"]


def ragged_workload(**over):
    # lengths around page and tile edges, one empty request
    w = I.Workload("ragged", seed=11, ctx_lens=[1, 63, 64, 65, 1000, 2049, 0, 4097],
                   num_layers=2, tile_tokens=1024)
    for k, v in over.items():
        setattr(w, k, v)
    return w


@pytest.fixture(scope="module")
def tiny(gpu):
    return Case(I.workload("tiny"))


@pytest.fixture(scope="module")
def ragged(gpu):
    return Case(ragged_workload(), fill=I.BF16_QNAN)


@pytest.mark.parametrize("kernel", KERNELS)
def test_tiny_partials_and_merge(tiny, kernel):
    """1 request x 4,096 tokens, tile 1,024: four partials and their merge."""
    got = tiny.decode(0, kernel=kernel)
    ref = tiny.oracle_layer(0)
    err = check_layer(tiny, 0, got, ref)
    print(f"tiny {kernel}: max abs err {err:.2e}")


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("tile,split", [(1024, 0), (256, 0), (2048, 64), (64, 0), (4096, 1024)])
def test_ragged_lengths(ragged, kernel, tile, split):
    """Lengths 0, 1, 63, 64, 65, 1000, 2049, 4097 on a NaN-poisoned arena,
    for tiles that are and are not one work-group's split."""
    for layer in (0, 1):
        got = ragged.decode(layer, tile=tile, kernel=kernel, split=split)
        ref = ragged.oracle_layer(layer, tile=tile)
        check_layer(ragged, layer, got, ref)


@pytest.mark.parametrize("kernel", KERNELS)
def test_run_to_run_and_staged_bitwise(ragged, kernel):
    """Reflexive control (two identical runs agree bit for bit), then staged
    windows of 2,048 tokens against one resident call at the same tiling."""
    a = ragged.decode(1, tile=512, kernel=kernel)
    b = ragged.decode(1, tile=512, kernel=kernel)
    for x, y in zip(a, b):
        assert same_bits(x, y)
    c = ragged.decode(1, tile=512, kernel=kernel, staged=2048)
    for x, y in zip(a, c):
        assert same_bits(x, y)


@pytest.mark.parametrize("kernel", KERNELS)
def test_poisoned_padding_and_placement(gpu, kernel):
    """Padding (NaN vs 0) and the physical placement of pages change no bit."""
    w = ragged_workload(num_layers=1)
    base = Case(w, fill=0)
    ref = base.decode(0, kernel=kernel)
    pois = Case(w, fill=I.BF16_QNAN)
    for x, y in zip(ref, pois.decode(0, kernel=kernel)):
        assert same_bits(x, y)
    perm = np.random.default_rng(99).permutation(w.num_pages).astype(np.int32)
    t2 = np.where(base.table >= 0, perm[np.maximum(base.table, 0)], -1).astype(np.int32)
    moved = Case(w, fill=I.BF16_QNAN, table=t2)
    for x, y in zip(ref, moved.decode(0, kernel=kernel)):
        assert same_bits(x, y)


def test_kernels_agree(ragged):
    """VALU and MFMA kernels agree with each other within the tolerance."""
    a = ragged.decode(0, tile=1024, kernel="valu")
    b = ragged.decode(0, tile=1024, kernel="mfma")
    assert torch.isneginf(a[3]).equal(torch.isneginf(b[3]))
    assert (a[2] - b[2]).abs().max().item() <= 2e-3


# ---------------------------------------------------------------- merge --


@pytest.fixture(scope="module")
def stress(gpu):
    """64 x 24 x 256 partials of width 256, lse ~ U[-40, 40], ~10 % empty,
    built by the oracle from explicit keys (4 per partial)."""
    d = I.stress_draws()
    o, lse, scores = oracle.stress_partials(d["r"], d["vals"], d["target_lse"], d["empty"])
    uo, ul = oracle.union_attention(scores, d["vals"])
    po = torch.from_numpy(o.astype(np.float32)).to(DEV)
    pl = torch.from_numpy(lse.astype(np.float32)).to(DEV)
    return po, pl, uo, ul


def merge(po, pl):
    from paged_kv_cache_10_amd import pkv
    rows = po.shape[:-2]
    out = torch.empty(rows + (po.shape[-1],), device=DEV)
    lse = torch.empty(rows, device=DEV)
    pkv.merge_partials(po, pl, out, lse)
    torch.cuda.synchronize()
    return out, lse


def test_merge_stress_matches_union_softmax(stress):
    po, pl, uo, ul = stress
    out, lse = merge(po, pl)
    assert_out_close(out.cpu().numpy(), uo)
    assert_lse_close(lse.cpu().numpy(), ul)
    # the forced rows: (0,0) all empty, (0,1) one live partial
    assert torch.all(out[0, 0] == 0) and lse[0, 0].item() == -math.inf
    live = int(np.flatnonzero(np.isfinite(pl[0, 1].cpu().numpy()))[0])
    assert same_bits(out[0, 1], po[0, 1, live]) and same_bits(lse[0, 1], pl[0, 1, live])


def test_merge_identity_and_empty_insertion_bitwise(stress):
    po, pl, _, _ = stress
    # one slot merges to itself, bit for bit
    o1, l1 = merge(po[:, :, 7:8].contiguous(), pl[:, :, 7:8].contiguous())
    live = torch.isfinite(pl[:, :, 7])
    assert same_bits(o1[live], po[:, :, 7][live]) and same_bits(l1[live], pl[:, :, 7][live])
    # inserting empty slots (lse = -inf, output NaN) changes no bit
    ref = merge(po, pl)
    S = po.shape[2]
    ins = [0, 5, 5, 100, S]
    parts_o, parts_l = [], []
    prev = 0
    for i in ins:
        parts_o.append(po[:, :, prev:i])
        parts_l.append(pl[:, :, prev:i])
        parts_o.append(torch.full_like(po[:, :, :1], float("nan")))
        parts_l.append(torch.full_like(pl[:, :, :1], -math.inf))
        prev = i
    got = merge(torch.cat(parts_o, 2).contiguous(), torch.cat(parts_l, 2).contiguous())
    for x, y in zip(ref, got):
        assert same_bits(x, y)


@pytest.mark.parametrize("n", [5, 64, 200])
def test_merge_nan_rows_match_the_oracle(stress, n):
    """A slot with a NaN log-sum-exp (a flagged partial) makes its row NaN,
    as the oracle's merge does; rows with only empty slots give (0, -inf);
    the other rows match the oracle.  Rows of at most 64 slots and longer
    rows take different merge kernels."""
    po, pl, _, _ = stress
    po, pl = po[:, :, :n].clone(), pl[:, :, :n].clone()
    pl[0, 2, n // 2] = float("nan")          # one flagged slot among live ones
    pl[1, 5, :] = float("-inf")              # every slot empty
    pl[1, 6, :] = float("-inf")
    pl[1, 6, n - 1] = float("nan")           # a flagged slot among empties
    out, lse = merge(po.contiguous(), pl.contiguous())
    eo, el = oracle.merge(po.cpu().numpy(), pl.cpu().numpy())
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    nan_rows = np.isnan(el)
    assert nan_rows[0, 2] and nan_rows[1, 6] and nan_rows.sum() == 2
    np.testing.assert_array_equal(np.isnan(l), nan_rows)
    assert np.isnan(o[nan_rows]).all()
    assert l[1, 5] == -math.inf and (o[1, 5] == 0).all()
    ok = ~nan_rows
    assert_out_close(o[ok], eo[ok], tol=1e-4)
    assert_lse_close(l[ok], el[ok])


@pytest.mark.parametrize("n", [1, 2, 17, 63, 64])
def test_merge_of_one_chunk_matches_two_chunks_bitwise(stress, n):
    """Rows of at most 64 slots are merged as one chunk of slots; the same
    slots followed by empty ones (more than 64 in all) take a second chunk.
    Empty slots contribute nothing, so the two must agree bit for bit; both
    against the float64 merge of the same FP32 partials."""
    po, pl, _, _ = stress
    po_n, pl_n = po[:, :, :n].contiguous(), pl[:, :, :n].contiguous()
    few = merge(po_n, pl_n)
    pad = 65 - n
    general = merge(torch.cat([po_n, torch.full_like(po[:, :, :pad], float("nan"))], 2).contiguous(),
                    torch.cat([pl_n, torch.full_like(pl[:, :, :pad], -math.inf)], 2).contiguous())
    for x, y in zip(few, general):
        assert same_bits(x, y)
    eo, el = oracle.merge(po_n.cpu().numpy(), pl_n.cpu().numpy())
    assert_out_close(few[0].cpu().numpy(), eo, tol=1e-4)
    assert_lse_close(few[1].cpu().numpy(), el, tol=1e-4)


@pytest.mark.parametrize("kernel", KERNELS)
def test_workspace_reuse_across_calls(ragged, kernel):
    """Tiles of 32 splits (2,048-token tiles of 64-token splits): three
    back-to-back calls on one workspace give the same bits as a fresh
    workspace each time."""
    from paged_kv_cache_10_amd import pkv
    w = ragged.w
    tile, split = 2048, 64
    S = ragged.num_slots(tile)
    fresh = [ragged.decode(layer, tile=tile, kernel=kernel, split=split) for layer in (0, 1, 0)]
    B, Hq, D = w.batch, w.num_q_heads, w.head_dim
    nbytes = pkv.decode_workspace_bytes(B, Hq, S * tile, tile, D, kernel, split)
    ws = torch.zeros(nbytes // 4 + 4, device=DEV)
    for layer, ref in zip((0, 1, 0), fresh):
        po = torch.empty((B, Hq, S, D), device=DEV)
        pl = torch.empty((B, Hq, S), device=DEV)
        pkv.decode_attention(ragged.pool, layer, ragged.q[layer], ragged.dev_table, ragged.dev_ctx,
                             0, S * tile, tile, w.scale, po, pl, workspace=ws, kernel=kernel,
                             split_tokens=split)
        torch.cuda.synchronize()
        assert same_bits(po, ref[0]) and same_bits(pl, ref[1])


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 4), (12, 4), (16, 4), (20, 4), (28, 4), (32, 4),
                                    (48, 4), (64, 4), (16, 2)])
def test_query_group_sizes(gpu, hq, hkv):
    """Query groups of 1, 2, 3, 4, 5, 7, 8, 12 and 16 heads per KV head (MFMA; the
    VALU kernel up to 8), against the oracle, lengths around page edges."""
    w = I.Workload("groups", seed=21, ctx_lens=[130, 2049, 777], num_layers=1,
                   tile_tokens=1024, num_q_heads=hq, num_kv_heads=hkv)
    case = Case(w, fill=I.BF16_QNAN)
    ref = case.oracle_layer(0)
    kernels = ["mfma"] + (["valu"] if hq // hkv <= 8 else [])
    for kernel in kernels:
        for split in (0, 256):
            check_layer(case, 0, case.decode(0, kernel=kernel, split=split), ref)


def test_one_million_tokens(gpu):
    """One request of 1,048,576 tokens (one layer, 4 GiB of KV), 1 % of keys
    scaled by 4, 4,096-token tiles: 256 partials per head merged in FP32."""
    w = I.Workload("long1m", seed=31, ctx_lens=[1 << 20], num_layers=1, tile_tokens=4096,
                   boost_frac=0.01)
    case = Case(w, host=False)
    got = case.decode(0, split=4096)
    err = check_layer(case, 0, got, case.oracle_layer(0))
    print(f"1M tokens: max abs err {err:.2e}")
    del case
    torch.cuda.empty_cache()
