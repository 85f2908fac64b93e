"""GPU: the C ABI used from C++ alone (tests/c_abi/decode_from_c.cpp, built
by the package build): pool, page tables, the history written with
pkv_append_kv, merged decode (checked there against decode + merge, and
against the asynchronous table write from pinned memory followed by the
no-allocation merged decode, bit for bit), and the results here against
the float64 oracle on the inputs the program wrote.  The program also runs
one live-pool step over a pinned host copy of the histories (sink and
newest pages resident, the rest staged, the last token appended again and
written back) and checks it bit for bit against the resident decode and the
host copy unchanged."""

import os
import subprocess

import numpy as np
import pytest

import oracle
from gpu_helpers import assert_lse_close, assert_out_close

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "decode_from_c")


def test_decode_through_the_c_abi_matches_oracle(gpu, tmp_path):
    assert os.path.exists(EXE), "build the package first (it builds the C-ABI test program)"
    out_file = tmp_path / "c_abi.bin"
    r = subprocess.run([EXE, str(out_file)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
    raw = out_file.read_bytes()
    off = 0

    def take(dtype, n):
        nonlocal off
        a = np.frombuffer(raw, dtype=dtype, count=n, offset=off)
        off += a.nbytes
        return a
    B, Hq, Hkv, D = take(np.int32, 4).tolist()
    ctx = take(np.int32, B).tolist()
    q = take(np.uint16, B * Hq * D).reshape(B, Hq, D)
    kv = []
    for b in range(B):
        k = take(np.uint16, Hkv * ctx[b] * D).reshape(Hkv, ctx[b], D)
        v = take(np.uint16, Hkv * ctx[b] * D).reshape(Hkv, ctx[b], D)
        kv.append((k, v))
    out = take(np.float32, B * Hq * D).reshape(B, Hq, D)
    lse = take(np.float32, B * Hq).reshape(B, Hq)
    assert off == len(raw)
    for b in range(B):
        k, v = kv[b]
        ro, rl = oracle.decode_one_pass(oracle.widen_bf16(q[b]), oracle.widen_bf16(k),
                                        oracle.widen_bf16(v), ctx[b], 1.0 / 16.0, Hkv)
        assert_out_close(out[b], ro)
        assert_lse_close(lse[b], rl)
