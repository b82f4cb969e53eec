import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line(
        "markers", "exhaustive: long exhaustive sweep, runs only with DUCKMOE_EXHAUSTIVE=1")


def pytest_collection_modifyitems(config, items):
    if os.environ.get("DUCKMOE_EXHAUSTIVE") == "1":
        return
    skip = pytest.mark.skip(reason="exhaustive sweep: set DUCKMOE_EXHAUSTIVE=1 to run")
    for item in items:
        if "exhaustive" in item.keywords:
            item.add_marker(skip)
