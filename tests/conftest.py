import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP C-ABI library)")
    config.addinivalue_line("markers", "slow: full-size workload")


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    # The oracle is cheap to compile; build it when the shared object is absent.
    path = os.path.join(ROOT, "oracle", "liboracle.so")
    if not os.path.exists(path):
        from oracle import build as b
        b.build()
    yield
