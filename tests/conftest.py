import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload, long-running")


@pytest.fixture(scope="session")
def hip():
    """The HIP library binding; a GPU test fails loudly if it is not built."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import differentiable_sparse_linear_amd as sla
    sla.load()  # raises if libsla.so is missing
    return sla
