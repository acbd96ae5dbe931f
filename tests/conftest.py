import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


@pytest.fixture(autouse=True)
def _announce(request):
    """Name each GPU case on stdout before it runs (flushed), so a run that
    dies on the GPU still says which case it was in."""
    if request.node.get_closest_marker("gpu") is not None:
        print(f"\n[gpu case] {request.node.nodeid}", flush=True)
    yield
