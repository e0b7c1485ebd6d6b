import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; calls the HIP library through its C ABI")


def _announce(item):
    # name the case before any GPU step so a lost box still says what ran
    sys.stderr.write(f"\n[case] {item.nodeid}\n")
    sys.stderr.flush()


@pytest.hookimpl(tryfirst=True)
def pytest_runtest_setup(item):
    if item.get_closest_marker("gpu") is not None:
        _announce(item)
