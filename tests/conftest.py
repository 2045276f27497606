import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running (full-size) test")


@pytest.fixture(scope="session")
def torch_cpu():
    import torch
    torch.set_num_threads(min(8, os.cpu_count() or 1))
    return torch
