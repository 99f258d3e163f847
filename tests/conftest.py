import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.dirname(os.path.abspath(__file__))
for p in (ROOT, TESTS):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle
    return oracle.load()


def pytest_runtest_logstart(nodeid, location):
    # Name the case on the real stderr before it runs, so that a run which
    # ends abruptly still shows which test (and so which shape) was on the GPU.
    if "gpu" in nodeid or "smoke" in nodeid:
        sys.__stderr__.write(f"[start] {nodeid}\n")
        sys.__stderr__.flush()
