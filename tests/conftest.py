import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload check (seconds to a minute)")


@pytest.fixture(scope="session")
def cuda_device():
    """The GPU the HIP tests run on; skips only when no GPU is present at all."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible to torch")
    return torch.device("cuda:0")
