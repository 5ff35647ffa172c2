import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running case")


@pytest.fixture(scope="session")
def gpu_lib():
    """The built HIP library on a visible GPU; fails loudly when either is missing."""
    import torch
    from adaptive_looped_denoising_amd import binding
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected without a visible GPU")
    return binding.load()
