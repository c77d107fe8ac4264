import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


import pytest


@pytest.fixture(scope="session")
def af():
    """The C-ABI binding; builds the library first if nothing is built."""
    import flow_matching_mmdit_amd as pkg
    if not os.path.exists(pkg.LIB_PATH):
        from flow_matching_mmdit_amd import build
        build.build()
    from flow_matching_mmdit_amd import binding
    return binding
