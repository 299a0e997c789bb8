import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes tens of seconds on the CPU")


def gpu_available() -> bool:
    import torch
    return torch.cuda.is_available()


@pytest.fixture(scope="session")
def require_gpu():
    if not gpu_available():
        pytest.skip("no GPU visible")
