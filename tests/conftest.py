import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session", autouse=True)
def _libraries_built():
    # Normally built beforehand by __graft_entry__.build(); build here only if absent.
    import oracle
    if not os.path.exists(oracle._LIB):
        oracle.build()
    from gemm_activation_reduction_amd import LIB_PATH, build
    if not os.path.exists(LIB_PATH):
        build.build()
    yield
