import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session", autouse=True)
def _gpu_runtime_first(request):
    """In a session that runs GPU tests, bring the HIP runtime up before any test runs: every
    GPU process then initialises it before the oracle's OpenMP threads exist."""
    if any(item.get_closest_marker("gpu") for item in request.session.items):
        import torch
        if torch.cuda.is_available():
            torch.empty(1, device="cuda:0")
            torch.cuda.synchronize()
    yield


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


def pytest_runtest_logstart(nodeid, location):
    # Name each test on the real stdout before it runs, so a run that dies mid-test says where.
    sys.__stdout__.write("\n[start] %s\n" % nodeid)
    sys.__stdout__.flush()
