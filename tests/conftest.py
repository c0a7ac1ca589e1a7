import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU-only exhaustive check (run with -m slow)")


def pytest_collection_modifyitems(config, items):
    # slow tests run only when asked for explicitly with -m slow
    markexpr = config.getoption("-m") or ""
    if "slow" in markexpr:
        return
    skip = pytest.mark.skip(reason="exhaustive check; run with -m slow")
    for item in items:
        if "slow" in item.keywords:
            item.add_marker(skip)
