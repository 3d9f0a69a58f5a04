import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the HIP library")


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    # The oracle is a plain C file; build it once if this tree has no copy yet.
    import oracle
    if not os.path.exists(oracle.lib_path()):
        oracle.build()
    yield
