import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (HIP device); parity tests proper")


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    """The CPU oracle is test infrastructure; build it if it is missing."""
    lib = os.path.join(ROOT, "oracle", "libgdr_oracle.so")
    if not os.path.exists(lib):
        from oracle import build
        build.build()
    yield
