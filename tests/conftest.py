import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: longer CPU test")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def gpu():
    # GPU tests never skip silently: on a machine without a GPU they are
    # deselected with -m "not gpu"; if selected, a missing GPU is a failure.
    if not gpu_available():
        pytest.fail("GPU test selected but no GPU is visible to torch")
    return True


@pytest.fixture(scope="session", autouse=True)
def built_library():
    """Build the HIP library if it is missing (it is not committed) or was
    built from other sources than the ones in the tree; a current build is
    used as it is."""
    from kv_cache_eviction_decode_amd.build import ensure_built
    ensure_built(verbose=True)
