import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libc3.so")


@pytest.fixture(scope="session")
def orc():
    """The CPU oracle (built with gcc on first use if liboracle.so is missing)."""
    import oracle

    oracle.lib()
    return oracle
