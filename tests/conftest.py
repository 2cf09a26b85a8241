import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU-only statistical test")


@pytest.fixture(scope="session")
def lores_lib():
    """liblores.so, built in-tree first if it is missing (hipcc cross-compiles on CPU)."""
    from quantized_linear_recurrence_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from quantized_linear_recurrence_amd import build
        build.build()
    return _lib.lib()
