import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library through its Python binding; GPU tests only."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected without a GPU")
    import mla_decode_paged_amd as mla
    mla.load()
    return mla
