import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line(
        "markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library on a visible GPU; the test fails loudly without it."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected but no GPU is visible")
    import rank_orthonormalized_optimizer_dion_amd as dion
    dion.load()   # raises if the HIP build is missing
    return dion
