import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")


@pytest.fixture(scope="session")
def gpu():
    """Skip when no GPU is visible; otherwise load the HIP library."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import exact_io_aware_44_amd as fa
    fa.load()  # raises if libfa.so is missing: there is no CPU fallback
    return fa
