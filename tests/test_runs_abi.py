"""pkv_decode_attention_runs on the host (no GPU): every argument check of
the one-launch decode of two runs, with fake pools whose arenas are never
dereferenced."""

import ctypes

import pytest

from paged_kv_cache_10_amd import pkv
from test_abi import FakeCompactPool, FakePool, err, geom


def run(pool, table=1 << 21, pt=512, ctx=1 << 22, count=32768, tile=4096, off=0):
    return pkv.DecodeRun(pool.handle if pool else None, table, pt, ctx, count, tile, off)


def call(runs, layer=0, q=1 << 20, batch=1, hq=24, scale=0.0625, po=1 << 23, pl=1 << 24,
         slots=16, n=None):
    arr = (pkv.DecodeRun * max(1, len(runs)))(*runs)
    rc = pkv.lib().pkv_decode_attention_runs(layer, q, batch, hq, arr if runs else None,
                                             len(runs) if n is None else n, scale, po, pl, slots,
                                             None)
    return rc, err()


@pytest.fixture(scope="module")
def pools():
    return FakeCompactPool(64), FakePool(64)


def test_two_valid_runs_pass_the_host_checks_with_no_requests(pools):
    c, e = pools
    rc, msg = call([run(c, count=28672, tile=4096), run(e, count=4096, tile=512, off=7)],
                   batch=0)
    assert rc == 0, msg


@pytest.mark.parametrize("kw,needle", [
    (dict(n=0), "n_runs"),
    (dict(n=3), "n_runs"),
    (dict(layer=16), "layer"),
    (dict(hq=25), "num_q_heads"),
    (dict(hq=4 * 9), "query group"),
    (dict(slots=0), "num_slots"),
    (dict(scale=float("inf")), "scale"),
    (dict(q=0), "NULL"),
    (dict(q=(1 << 20) + 2), "aligned"),
])
def test_call_arguments_are_refused(pools, kw, needle):
    c, e = pools
    rc, msg = call([run(c, count=28672, tile=4096), run(e, count=4096, tile=512, off=7)], **kw)
    assert rc != 0 and needle in msg, msg


@pytest.mark.parametrize("k,kw,needle", [
    (0, dict(tile=100), "tile_tokens"),
    (0, dict(tile=32768), "tile_tokens"),
    (1, dict(count=1000), "token_count"),
    (1, dict(pt=4), "pt_stride"),
    (1, dict(off=14), "num_slots"),
    (1, dict(off=6), "overlap"),
    (0, dict(table=0), "dev_table"),
    (1, dict(ctx=0), "dev_ctx_lens"),
])
def test_run_arguments_are_refused(pools, k, kw, needle):
    c, e = pools
    runs = [dict(pool=c, count=28672, tile=4096), dict(pool=e, count=4096, tile=512, off=7)]
    runs[k].update(kw)
    rc, msg = call([run(**r) for r in runs])
    assert rc == -1 and needle in msg, msg
    if needle != "overlap":
        assert f"runs[{k}]" in msg, msg


def test_null_pool_and_mismatched_heads_are_refused(pools):
    c, e = pools
    rc, msg = call([run(None)])
    assert rc == -1 and "runs[0].pool" in msg
    h = pkv.P()
    assert pkv.lib().pkv_pool_create(ctypes.byref(geom(hkv=8)), 1 << 20,
                                     pkv.page_bytes(16, 8) * 8, ctypes.byref(h)) == 0
    try:
        rc, msg = call([run(c, count=28672, tile=4096),
                        pkv.DecodeRun(h, 1 << 21, 512, 1 << 22, 4096, 512, 7)])
        assert rc == -3 and "KV heads" in msg
    finally:
        pkv.lib().pkv_pool_destroy(h)
