import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (minutes of host work)")


def gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def gpu():
    """The HIP binding, loaded; skips the test when no GPU is visible."""
    if not gpu_available():
        pytest.skip("no GPU visible")
    from paged_kv_cache_10_amd import pkv
    pkv.lib()          # raises if libpkv.so is missing: no silent fallback
    return pkv
