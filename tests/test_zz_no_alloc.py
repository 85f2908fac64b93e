"""pkv_decode_attention_merged_noalloc on the GPU, through the C ABI: the
split partials of each tile live in the library's static device scratch
instead of a caller workspace.  Two calls in a row, the second on a smaller
input, each give the same bits as pkv_decode_attention_merged with a
workspace (the same kernels), and match the oracle."""

import numpy as np
import pytest
import torch

from paged_kv_cache_10_amd import inputs as I
from paged_kv_cache_10_amd import pkv
from gpu_helpers import Case, DEV, check_layer, same_bits

pytestmark = pytest.mark.gpu


def run(case, tile, split, noalloc):
    w = case.w
    S = case.num_slots(tile)
    B, Hq, D = w.batch, w.num_q_heads, w.head_dim
    po = torch.full((B, Hq, S, D), float("nan"), device=DEV)
    pl = torch.full((B, Hq, S), float("nan"), device=DEV)
    o = torch.full((B, Hq, D), float("nan"), device=DEV)
    l = torch.full((B, Hq), float("nan"), device=DEV)
    if noalloc:
        pkv.decode_attention_merged_noalloc(case.pool, 0, case.q[0], case.dev_table, case.dev_ctx,
                                            S * tile, tile, w.scale, po, pl, o, l,
                                            split_tokens=split)
    else:
        nb = pkv.decode_workspace_bytes(B, Hq, S * tile, tile, D, 0, split)
        ws = torch.zeros(max(nb, 16) // 4 + 4, dtype=torch.float32, device=DEV)
        pkv.decode_attention_merged(case.pool, 0, case.q[0], case.dev_table, case.dev_ctx,
                                    S * tile, tile, w.scale, po, pl, o, l, workspace=ws,
                                    split_tokens=split)
    torch.cuda.synchronize()
    return po, pl, o, l


def test_noalloc_equals_the_workspace_call_twice_in_a_row(gpu):
    big = Case(I.Workload("noalloc", seed=71, ctx_lens=[20000, 9000, 500, 16384], num_layers=1,
                          tile_tokens=8192))
    small = Case(I.Workload("noalloc", seed=72, ctx_lens=[3000], num_layers=1, tile_tokens=4096))
    for case, tile, split in ((big, 8192, 2048), (small, 4096, 1024)):
        need = pkv.decode_workspace_bytes(case.w.batch, case.w.num_q_heads,
                                          case.num_slots(tile) * tile, tile, 256, 0, split)
        assert 0 < need <= pkv.STATIC_SCRATCH_BYTES
        got = run(case, tile, split, noalloc=True)
        ref = run(case, tile, split, noalloc=False)
        for x, y in zip(got, ref):
            assert same_bits(x, y), (case.w.ctx_lens, tile)
        check_layer(case, 0, got, case.oracle_layer(0, tile=tile))
