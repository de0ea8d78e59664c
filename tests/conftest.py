import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) HIP device")
    config.addinivalue_line("markers", "slow: long CPU check, skipped unless --runslow")


def pytest_addoption(parser):
    parser.addoption("--runslow", action="store_true", default=False, help="run slow CPU checks")


def pytest_collection_modifyitems(config, items):
    import pytest

    if config.getoption("--runslow"):
        return
    skip = pytest.mark.skip(reason="slow CPU check: pass --runslow")
    for item in items:
        if "slow" in item.keywords:
            item.add_marker(skip)
