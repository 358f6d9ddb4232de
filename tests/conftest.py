import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.build()
    return oracle


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    """Name each GPU test on the real stderr before it touches the device."""
    if request.node.get_closest_marker("gpu") is not None:
        from helpers import announce
        announce(request.node.nodeid)
    yield


@pytest.fixture(scope="session")
def dsa():
    import sparse_attention_09_amd as d
    d.lib()  # fails loudly if libdsa.so is missing
    return d
