import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size parity case")


import pytest  # noqa: E402


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    """Name each GPU case on stderr (uncaptured, flushed) before it runs."""
    if request.node.get_closest_marker("gpu"):
        sys.__stderr__.write(f"[gpu-case] {request.node.nodeid}\n")
        sys.__stderr__.flush()
    yield
