import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    """Name each GPU test on stderr before it runs, so a failure that takes the
    process down still says which case it was."""
    if request.node.get_closest_marker("gpu") is not None:
        sys.stderr.write(f"\n[gpu case] {request.node.nodeid}\n")
        sys.stderr.flush()
    yield
