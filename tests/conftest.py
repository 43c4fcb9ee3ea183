import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")
    config.addinivalue_line("markers", "fullsize: GPU parity case at a full K3 layer size (runs after the small cases)")


def pytest_collection_modifyitems(config, items):
    # Full-size GPU cases run after the small ones, so that a failure in a late, heavy
    # case does not hide the small parity cases before it; the entry point that
    # allocates nothing (test_zz_no_alloc.py) is checked after everything else.
    def order(it):
        if os.path.basename(str(it.fspath)) == "test_zz_no_alloc.py":
            return 2
        return 1 if it.get_closest_marker("fullsize") else 0
    items.sort(key=order)
