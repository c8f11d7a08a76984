import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long CPU sweep")


GPU_TEST_TIMEOUT_S = 300  # the longest GPU test takes well under a minute


def pytest_collection_modifyitems(config, items):
    """Every GPU test without a timeout of its own gets one (when the
    pytest-timeout plugin is there), enforced from a watchdog thread, which
    can end a test that is waiting inside a GPU call: a run without
    --timeout then still ends, naming the test, instead of waiting forever."""
    if not config.pluginmanager.hasplugin("timeout"):
        return
    for item in items:
        if item.get_closest_marker("gpu") and not item.get_closest_marker("timeout"):
            item.add_marker(pytest.mark.timeout(GPU_TEST_TIMEOUT_S, method="thread"))


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.fixture
def golden():
    return load_golden
