"""Shared test configuration.

Marker `gpu`: the test needs an MI355X (HIP device) and the built library.
Everything else runs on the host without a GPU.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a HIP GPU and the built libulysses.so")


@pytest.fixture(scope="session")
def golden():
    import json
    with open(os.path.join(ROOT, "tests", "golden", "pages_examples.json")) as f:
        return json.load(f)
