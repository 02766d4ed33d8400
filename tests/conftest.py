import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests load the in-tree library; build it only if nothing is built.
    if any(item.get_closest_marker("gpu") for item in items):
        from kimi_delta_attention_amd import _lib
        if not os.path.exists(_lib.LIB_PATH):
            from kimi_delta_attention_amd import build
            build.build()


GOLDEN = os.path.join(TESTS, "golden")


@pytest.fixture(scope="session")
def golden_dir():
    return GOLDEN
