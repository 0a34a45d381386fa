import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library through its Python binding; fails loudly if absent."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import long_context_sparse_head_amd as rtp
    rtp.load()  # raises if librtp.so is missing
    return rtp
