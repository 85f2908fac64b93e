"""Build libpkv.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m paged_kv_cache_10_amd.build [--resource-usage]

Also builds ``probe_read``, a standalone HBM read-ceiling probe, and
``tests/c_abi/decode_from_c``, the test program that drives the C ABI from
C++ alone.
Every source is compiled by hipcc with packed-FP32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``), objects go to
``_build/`` and the shared library lands next to this file.
"""

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpkv.so")
PROBE = os.path.join(HERE, "probe_read")          # HBM read-ceiling probe (an executable)
C_ABI_SRC = os.path.join(os.path.dirname(HERE), "tests", "c_abi", "decode_from_c.cpp")
C_ABI_EXE = os.path.join(os.path.dirname(HERE), "tests", "c_abi", "decode_from_c")
ARCH = "gfx950"

SOURCES = ["api.cpp", "stager.cpp", "admit.cpp", "live.cpp", "merge.hip", "decode_valu.hip", "decode_mfma.hip", "append.hip", "compact.hip", "decode_fp8.hip", "decode_runs.hip"]

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
    f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found (ROCm is required to build libpkv)")
    return exe


def _compile(src, resource_usage):
    obj = os.path.join(BUILD, src + ".o")
    cmd = [hipcc()] + COMMON + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if resource_usage and src.endswith(".hip"):
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    p = subprocess.run(cmd, capture_output=True, text=True)
    return src, obj, p.returncode, p.stdout + p.stderr


def build(resource_usage=False, verbose=False):
    """Compile every source and link libpkv.so; raises on any error."""
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    logs = []
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        for src, obj, rc, out in ex.map(lambda s: _compile(s, resource_usage), SOURCES):
            # the host pass does not know the packed-fp32 target feature: harmless
            out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{out}")
            if out.strip():
                logs.append(f"== {src}\n{out}")
            objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed:\n{p.stdout}{p.stderr}")
    os.replace(tmp, LIB)
    cmd = [hipcc()] + COMMON + [os.path.join(CSRC, "probe_read.hip"), "-o", PROBE + ".tmp"]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"probe build failed:\n{p.stdout}{p.stderr}")
    os.replace(PROBE + ".tmp", PROBE)
    # the C-ABI test program (tests/c_abi): the library used from C++ alone
    cmd = [hipcc(), "-O2", "-std=c++17", f"--offload-arch={ARCH}", "-x", "hip", C_ABI_SRC,
           "-o", C_ABI_EXE + ".tmp", "-L", HERE, "-lpkv",
           "-Wl,-rpath,$ORIGIN/../../paged_kv_cache_10_amd"]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"C-ABI test program build failed:\n{p.stdout}{p.stderr}")
    os.replace(C_ABI_EXE + ".tmp", C_ABI_EXE)
    if verbose or resource_usage:
        for l in logs:
            print(l)
    return LIB


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--resource-usage", action="store_true")
    args = ap.parse_args()
    print(build(resource_usage=args.resource_usage, verbose=True))


if __name__ == "__main__":
    sys.exit(main())
