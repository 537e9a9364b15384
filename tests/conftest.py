import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU oracle runs")


def gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def lib():
    """The HIP library through its Python binding; a GPU test without it fails
    loudly rather than falling back to anything."""
    if not gpu_available():
        pytest.fail("gpu test collected on a machine without a GPU")
    import mixture_experts_decode_amd as moe
    moe.load()
    return moe
