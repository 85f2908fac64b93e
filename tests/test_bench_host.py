"""CPU: the host-side rules of bench.py that decide what its JSON line may
claim (no GPU needed).

  * counter-derived traffic is reported only for the kernel sources and
    launch shapes the counters were taken on (null after any change to
    those sources), and is within 1 % of the algorithmic bytes there;
  * a request for more than one GPU is refused with a message, before
    anything touches a device."""

import os
import subprocess
import sys

import pytest

import bench
from paged_kv_cache_10_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def kv_bytes_per_layer(name):
    w = I.workload(name)
    return w.kv_bytes_per_step // w.num_layers


def counters_current():
    """True while every kernel source the counters were taken on is unchanged
    (after a change bench.py reports traffic as null until they are retaken)."""
    return (bench.sources_sha256(bench.KERNEL_SOURCES) == bench.PMC_TRAFFIC["source_sha256"]
            and bench.sources_sha256(bench.CONC_SOURCES) == bench.PMC_TRAFFIC_CONC["source_sha256"]
            and bench.PMC_TRAFFIC_MIXED["source_sha256"] == bench.PMC_TRAFFIC["source_sha256"])


def test_traffic_only_for_measured_shapes():
    if not counters_current():
        pytest.skip("kernel sources changed since the counters were taken: traffic is null")
    assert bench.pmc_traffic("long262k", 4096, 4096, "mfma") is not None
    assert bench.pmc_traffic("long262k", 4096, 2048, "mfma") is None      # another split
    assert bench.pmc_traffic("long262k", 4096, 4096, "valu") is None      # another kernel
    assert bench.pmc_traffic("conc", 8192, 2048, "mfma") is not None
    assert bench.pmc_traffic("conc", 8192, 1024, "mfma") is None
    assert bench.pmc_traffic("mixed", 4096, 4096, "mfma", plan=256) is not None
    assert bench.pmc_traffic("mixed", 4096, 4096, "mfma", plan=512) is None
    assert bench.pmc_traffic("mixed", 4096, 4096, "mfma") is None          # fixed tiling


def test_traffic_close_to_algorithmic_bytes():
    if not counters_current():
        pytest.skip("kernel sources changed since the counters were taken: traffic is null")
    for name, tile, split, plan in (("long262k", 4096, 4096, 0), ("conc", 8192, 2048, 0),
                                    ("mixed", 4096, 4096, 256)):
        ratio = bench.pmc_traffic(name, tile, split, "mfma", plan) / kv_bytes_per_layer(name)
        assert 1.0 <= ratio < 1.01, (name, ratio)


def test_traffic_dropped_when_the_kernel_source_changes(monkeypatch):
    monkeypatch.setattr(bench, "sources_sha256", lambda files: "0" * 64)
    assert bench.pmc_traffic("long262k", 4096, 4096, "mfma") is None
    assert bench.pmc_traffic("conc", 8192, 2048, "mfma") is None
    assert bench.pmc_traffic("mixed", 4096, 4096, "mfma", plan=256) is None


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert p.returncode != 0
    assert "one GPU" in (p.stdout + p.stderr)


def test_code_hash_ignores_comments_but_not_code(tmp_path):
    """The counters stay valid through a comment edit and are dropped by any
    change to the code, including inside a string literal."""
    src = tmp_path / "k.hip"
    base = 'int f(int x) {  // add one\n  return x + 1; /* done */\n}\nconst char* s = "a // b";\n'
    variants = {
        "comment": 'int f(int x) {  // add one to x\n  return x + 1;   /* finished\n */\n}\n'
                   'const char* s = "a // b";\n',
        "code": 'int f(int x) {  // add one\n  return x + 2; /* done */\n}\nconst char* s = "a // b";\n',
        "string": 'int f(int x) {  // add one\n  return x + 1; /* done */\n}\nconst char* s = "a // c";\n',
    }
    src.write_text(base)
    h0 = bench.sources_sha256(["k.hip"], root=str(tmp_path))
    got = {}
    for name, text in variants.items():
        src.write_text(text)
        got[name] = bench.sources_sha256(["k.hip"], root=str(tmp_path)) == h0
    assert got == {"comment": True, "code": False, "string": False}
