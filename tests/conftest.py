import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running full-size case")


@pytest.fixture(scope="session")
def gpu_lib():
    """The loaded C-ABI library (skips cleanly only when no GPU is visible)."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from dynamic_column_sparse_amd import lib
    return lib
