import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU case")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library through its Python binding; the test fails (not skips) if the
    library cannot be loaded on a GPU host."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_attention_43_amd import pisa
    pisa.load()          # raises if the shared library is missing
    return pisa
