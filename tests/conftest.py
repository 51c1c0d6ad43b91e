import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: takes more than a few seconds")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    return oracle.load()


def pytest_runtest_setup(item):
    # name a GPU case on the real stderr before it runs, so a run that dies on
    # the GPU still says which case it was in
    if item.get_closest_marker("gpu"):
        sys.__stderr__.write(f"[start] {item.nodeid}\n")
        sys.__stderr__.flush()
