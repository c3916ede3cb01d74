import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workloads (minutes of CPU oracle time)")


class T:
    """Minimal tensor record (type, rows, cols, raw bytes) for hand-built inputs."""

    def __init__(self, name, type, rows, cols, data):
        self.name, self.type, self.rows, self.cols, self.data = name, type, rows, cols, data


@pytest.fixture
def tensor_record():
    return T
