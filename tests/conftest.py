import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    """Name each GPU case on stdout (flushed) before it touches the device."""
    if request.node.get_closest_marker("gpu") is not None:
        print(f"\n[gpu case] {request.node.nodeid}", flush=True)
    yield
