import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workloads (minutes of CPU/GPU work)")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library through its Python binding; fails loudly if missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("a GPU test ran without a visible GPU")
    from lm_head_projection_amd import _lib
    return _lib.load()
