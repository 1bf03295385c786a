import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large workload, several seconds or more")


@pytest.fixture(scope="session")
def gpu_lib():
    """The loaded HIP library; fails loudly when the extension or the GPU is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("gpu test selected but torch.cuda.is_available() is False")
    import mixture_experts_top_amd as m
    m.load_library()
    return m
