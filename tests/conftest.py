import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


@pytest.fixture(scope="session")
def gpu_lib():
    """The built HIP library on a visible GPU; GPU tests fail loudly without it."""
    import torch
    import decode_attention_amd as da
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected on a machine without a GPU")
    da.load_library()  # raises if the shared library is missing
    return da
