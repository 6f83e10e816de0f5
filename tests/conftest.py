import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU check")


import pytest  # noqa: E402


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    """Name each GPU case on the real stderr before it touches the device, so
    a run that dies mid-test still says which case it was."""
    if request.node.get_closest_marker("gpu") is not None:
        sys.__stderr__.write("\n[gpu case] %s\n" % request.node.nodeid)
        sys.__stderr__.flush()
    yield
