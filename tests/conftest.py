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
    # GPU tests are collected last within the gpu selection so that a failure in a
    # late, heavy full-size case does not hide the small parity cases before it.
    items.sort(key=lambda it: 1 if it.get_closest_marker("fullsize") else 0)
