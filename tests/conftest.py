import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running check")


@pytest.fixture(scope="session")
def gpu_lib():
    """The C-ABI binding on cuda:0; GPU tests fail loudly if the library is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but no GPU is visible")
    from exact_io_aware_71_amd import binding
    binding.load()  # raises if libexact_attn.so is not built
    return binding
