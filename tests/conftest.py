import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long CPU-side work")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def lib():
    """The built C-ABI library (built first if no build is present)."""
    from w4a4_quantized_linear_cube_amd import dq
    if not os.path.exists(dq.library_path()):
        import __graft_entry__
        __graft_entry__.build()
    return dq.load()
