import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library binding; fails loudly if the GPU or the library is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    import block_sparse_attention_mask_amd as bsa
    bsa.load()          # raises if the shared library is not built
    return bsa
