import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line(
        "markers", "exhaustive: exhaustive sweep (about a minute on 8 cores); "
        "DUCKMOE_QUICK=1 skips it")


def pytest_collection_modifyitems(config, items):
    if os.environ.get("DUCKMOE_QUICK") != "1":
        return
    skip = pytest.mark.skip(reason="exhaustive sweep skipped (DUCKMOE_QUICK=1)")
    for item in items:
        if "exhaustive" in item.keywords:
            item.add_marker(skip)
