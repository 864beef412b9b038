import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def built_library():
    """The in-tree libpsgd.so, compiled with hipcc first if it is missing (hipcc
    cross-compiles gfx950 without a GPU).  A library that neither exists nor builds is
    an error of every test that asks for it, never a skip."""
    from distributed_sgd_gradient_ef_amd import build, psgd

    if not os.path.exists(psgd.LIB_PATH):
        build.build()
    return psgd.load_library()
