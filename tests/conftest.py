import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) HIP device")
    config.addinivalue_line("markers", "slow: larger CPU cases")


def gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


@pytest.fixture(scope="session")
def dev():
    """The HIP device for parity tests; the library must be built and load."""
    if not gpu_available():
        pytest.skip("no HIP device in this process")
    import torch
    import paged_kv_cache_204_amd as pkv
    pkv.load()          # raises if the built library is missing
    return torch.device("cuda:0")
