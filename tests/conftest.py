import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


def pytest_sessionstart(session):
    # The tests load the built library; build it (hipcc, gfx950) only when
    # it is missing, as in a fresh checkout.
    from top_reduce_amd import _binding, build
    if not os.path.exists(_binding.lib_path()):
        build.build()


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    return oracle
