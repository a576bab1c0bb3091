import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD Instinct GPU (gfx950) and the built HIP library")


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    import oracle
    src = os.path.join(ROOT, "oracle", "oracle.c")
    lib = os.path.join(ROOT, "oracle", "liboracle.so")
    if not os.path.exists(lib) or os.path.getmtime(lib) < os.path.getmtime(src):
        oracle.build()
    yield
