"""The live pool's host-side checks (pkv_live_*), on the CPU: every refusal
below happens before any HIP call, so no device is needed."""

import ctypes

import pytest

from paged_kv_cache_10_amd import pkv
from test_abi import FakePool, err


def create(pool, stage, host=1 << 30, host_bytes=None, max_batch=4, pt_stride=512,
           state=1 << 28):
    h = pkv.P()
    if host_bytes is None:
        host_bytes = pkv.page_bytes(16, 4) * 8
    rc = pkv.lib().pkv_live_create(pool.handle if pool else None, stage.handle if stage else None,
                                   host, host_bytes, max_batch, pt_stride, state, None, None,
                                   None, ctypes.byref(h))
    return rc, err()


@pytest.mark.parametrize("kw,needle", [
    (dict(pool=None), "NULL"),
    (dict(host=None), "host_arena"),
    (dict(state=None), "dev_state"),
    (dict(host_bytes=0), "host_bytes"),
    (dict(host_bytes=pkv.page_bytes(16, 4) * 8 + 1), "whole number"),
    (dict(max_batch=0), "max_batch"),
    (dict(pt_stride=0), "pt_stride"),
])
def test_create_arguments_are_refused_on_the_host(kw, needle):
    args = dict(pool=FakePool(64), stage=FakePool(64, layers=2))
    args.update(kw)
    rc, msg = create(**args)
    assert rc == -1 and needle in msg, msg


def test_staging_pool_with_other_heads_is_refused():
    L = pkv.lib()
    g = pkv.Geom(2, 8, 256, 64)
    h = pkv.P()
    assert L.pkv_pool_create(ctypes.byref(g), 1 << 30, pkv.page_bytes(2, 8) * 4, ctypes.byref(h)) == 0
    other = type("P", (), {"handle": h})()
    rc, msg = create(FakePool(64), other)
    assert rc == -3 and "KV heads" in msg
    L.pkv_pool_destroy(h)


def test_calls_on_no_runtime_are_refused():
    L = pkv.lib()
    assert L.pkv_live_add(None, 0, 4, 0) == -1
    assert L.pkv_live_remove(None, 0) == -1
    st = (ctypes.c_int32 * 1)()
    assert L.pkv_live_step_begin(None, 1, None, None, None, 1, st, None) == -1
    assert L.pkv_live_layer(None, 0, None, None, None, 24, 1024, 0.0625, None, None, 1, None,
                            None, None, 0, None) == -1
    assert L.pkv_live_attach_compact(None, None, None, 0, 1024, None) == -1
    pages = (ctypes.c_int32 * 1)(0)
    assert L.pkv_live_publish(None, pages, 1) == -1
    assert L.pkv_live_retract(None, pages, 1) == -1
    assert L.pkv_live_destroy(None) == 0
