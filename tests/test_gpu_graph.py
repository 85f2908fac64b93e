"""GPU: a decode step of several layers captured in a HIP graph
(torch.cuda.CUDAGraph) and replayed.  The decode and merge calls only
launch kernels on the caller's stream (no device allocation, no host
synchronisation, no memset), so a caller can capture them; every replay,
with the program's own eager work and synchronisations between replays, must
give the eager step's bits, and the eager step matches the float64 oracle.

Forms captured: decode + merge per layer (tiles that are splits, and tiles
finalized from smaller splits), the merged call with a workspace and the
one that allocates nothing, per-request tiles + merge, and compact + exact
runs in one launch + merge."""

import numpy as np
import pytest
import torch

from paged_kv_cache_10_amd import inputs as I
from paged_kv_cache_10_amd import pkv
from gpu_helpers import DEV, Case, Runs, check_layer, same_bits

pytestmark = pytest.mark.gpu

LAYERS = 2
REPLAYS = 3


@pytest.fixture(scope="module")
def case(gpu):
    w = I.Workload("graph", seed=21, ctx_lens=[5000, 1, 2049, 0, 3001], num_layers=LAYERS,
                   tile_tokens=1024)
    return Case(w, fill=I.BF16_QNAN)


def _buffers(case, slots):
    w = case.w
    B, Hq, D = w.batch, w.num_q_heads, w.head_dim
    po = [torch.empty((B, Hq, slots, D), device=DEV) for _ in range(LAYERS)]
    pl = [torch.empty((B, Hq, slots), device=DEV) for _ in range(LAYERS)]
    o = [torch.empty((B, Hq, D), device=DEV) for _ in range(LAYERS)]
    l = [torch.empty((B, Hq), device=DEV) for _ in range(LAYERS)]
    return po, pl, o, l


def _capture_and_replay(step, outputs):
    """Eager step on a side stream; the same step captured; REPLAYS replays,
    each after the outputs are poisoned and unrelated eager work has run.
    Returns the eager outputs (copies)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        for t in outputs:
            t.fill_(float("nan"))
        noise = torch.randn(1 << 20, device=DEV)
        noise.mul_(2.0).sum().item()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (t, e) in enumerate(zip(outputs, ref)):
            assert same_bits(t, e), f"replay {r}: output {i} differs from the eager step"
    del g
    torch.cuda.synchronize()
    return ref


def _check_eager(case, ref, tile):
    po, pl, o, l = ref
    for layer in range(LAYERS):
        check_layer(case, layer, (po[layer], pl[layer], o[layer], l[layer]),
                    case.oracle_layer(layer, tile=tile))


@pytest.mark.parametrize("tile,split", [(1024, 1024), (1024, 256)])
def test_graph_decode_then_merge(case, tile, split):
    w = case.w
    S = case.num_slots(tile)
    po, pl, o, l = _buffers(case, S)
    nb = pkv.decode_workspace_bytes(w.batch, w.num_q_heads, S * tile, tile, w.head_dim, 0, split)
    ws = torch.zeros(max(nb, 16) // 4 + 4, device=DEV)

    def step():
        for layer in range(LAYERS):
            pkv.decode_attention(case.pool, layer, case.q[layer], case.dev_table, case.dev_ctx,
                                 0, S * tile, tile, w.scale, po[layer], pl[layer], workspace=ws,
                                 split_tokens=split)
            pkv.merge_partials(po[layer], pl[layer], o[layer], l[layer])

    ref = _capture_and_replay(step, po + pl + o + l)
    n = LAYERS
    _check_eager(case, (ref[:n], ref[n:2 * n], ref[2 * n:3 * n], ref[3 * n:]), tile)


def test_graph_merged(case):
    w = case.w
    tile, split = 1024, 256
    S = case.num_slots(tile)
    po, pl, o, l = _buffers(case, S)
    nb = pkv.decode_workspace_bytes(w.batch, w.num_q_heads, S * tile, tile, w.head_dim, 0, split)
    ws = torch.zeros(max(nb, 16) // 4 + 4, device=DEV)

    def step():
        for layer in range(LAYERS):
            pkv.decode_attention_merged(case.pool, layer, case.q[layer], case.dev_table,
                                        case.dev_ctx, S * tile, tile, w.scale, po[layer],
                                        pl[layer], o[layer], l[layer], workspace=ws,
                                        split_tokens=split)

    ref = _capture_and_replay(step, po + pl + o + l)
    n = LAYERS
    _check_eager(case, (ref[:n], ref[n:2 * n], ref[2 * n:3 * n], ref[3 * n:]), tile)
    # the merged call's bits are those of decode then merge
    for layer in range(LAYERS):
        sep = case.decode(layer, tile=tile, split=split)
        for x, y in zip(sep, (ref[layer], ref[n + layer], ref[2 * n + layer], ref[3 * n + layer])):
            assert same_bits(x, y)


def test_graph_merged_noalloc(case):
    """The merged call that allocates nothing (split partials in the
    library's static scratch), captured and replayed: the bits of the
    workspace form, which the eager step checks against the oracle."""
    w = case.w
    tile, split = 1024, 256
    S = case.num_slots(tile)
    po, pl, o, l = _buffers(case, S)

    def step():
        for layer in range(LAYERS):
            pkv.decode_attention_merged_noalloc(case.pool, layer, case.q[layer], case.dev_table,
                                                case.dev_ctx, S * tile, tile, w.scale, po[layer],
                                                pl[layer], o[layer], l[layer], split_tokens=split)

    ref = _capture_and_replay(step, po + pl + o + l)
    n = LAYERS
    _check_eager(case, (ref[:n], ref[n:2 * n], ref[2 * n:3 * n], ref[3 * n:]), tile)
    nb = pkv.decode_workspace_bytes(w.batch, w.num_q_heads, S * tile, tile, w.head_dim, 0, split)
    ws = torch.zeros(max(nb, 16) // 4 + 4, device=DEV)
    for layer in range(LAYERS):
        got = [torch.empty_like(x) for x in (po[layer], pl[layer], o[layer], l[layer])]
        pkv.decode_attention_merged(case.pool, layer, case.q[layer], case.dev_table, case.dev_ctx,
                                    S * tile, tile, w.scale, *got, workspace=ws,
                                    split_tokens=split)
        torch.cuda.synchronize()
        for x, y in zip(got, (ref[layer], ref[n + layer], ref[2 * n + layer],
                              ref[3 * n + layer])):
            assert same_bits(x, y)


def test_graph_rows(case):
    w = case.w
    row_tiles, max_tiles = pkv.plan_tiles(w.ctx_lens, w.num_kv_heads, work_groups=64)
    po, pl, o, l = _buffers(case, max_tiles)
    dev_rt = torch.from_numpy(np.asarray(row_tiles, np.int32)).to(DEV)
    mrt = int(np.max(row_tiles))

    def step():
        for layer in range(LAYERS):
            pkv.decode_attention_rows(case.pool, layer, case.q[layer], case.dev_table,
                                      case.dev_ctx, dev_rt, mrt, max_tiles, w.scale, po[layer],
                                      pl[layer])
            pkv.merge_partials(po[layer], pl[layer], o[layer], l[layer])

    ref = _capture_and_replay(step, po + pl + o + l)
    n = LAYERS
    for layer in range(LAYERS):
        check_layer(case, layer, (ref[layer], ref[n + layer], ref[2 * n + layer],
                                  ref[3 * n + layer]),
                    case.oracle_rows(layer, row_tiles, max_tiles))


def test_graph_runs_one_launch(case):
    w = case.w
    runs = Runs(case, [4992, 0, 1984, 0, 2944])
    tile, etile = 1024, 512
    Sc, Se = runs.slots(tile, etile)
    po, pl, o, l = _buffers(case, Sc + Se)

    def step():
        for layer in range(LAYERS):
            pkv.decode_attention_runs(
                layer, case.q[layer],
                [(runs.pool, runs.dev_ct, runs.dev_cc, Sc * tile, tile, 0),
                 (case.pool, runs.dev_et, runs.dev_ec, Se * etile, etile, Sc)],
                w.scale, po[layer], pl[layer])
            pkv.merge_partials(po[layer], pl[layer], o[layer], l[layer])

    ref = _capture_and_replay(step, po + pl + o + l)
    n = LAYERS
    for layer in range(LAYERS):
        eager = runs.decode(layer, tile, etile=etile, one_launch=True)
        got = (ref[layer], ref[n + layer], ref[2 * n + layer], ref[3 * n + layer])
        for x, y in zip(eager, got):
            assert same_bits(x, y)
        runs.check(got, runs.oracle(layer, tile, etile=etile))
