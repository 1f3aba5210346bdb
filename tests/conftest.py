import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a GPU (runs the HIP path through the C ABI)")


@pytest.fixture(scope="session")
def orc():
    """The CPU oracle (built on first use)."""
    from oracle import build, ref
    if not os.path.exists(build.LIB):
        build.build()
    return ref
