import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: runs HIP kernels on an MI355X through the C-ABI library")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    oracle._load()
    return oracle
