import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: runs HIP kernels through the C-ABI on an MI355X")


@pytest.fixture(scope="session")
def gpu():
    """The HIP library on cuda:0. On a host without a GPU the test is skipped;
    on a host with one, a missing or unloadable library is an error."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this host")
    import zero_distributed_optimizer_amd as zdo
    zdo.require_library()
    return zdo
