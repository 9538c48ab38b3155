"""Shared pytest setup: the ``gpu`` marker and the one-time build of missing libraries."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs a real MI355X (gfx950); runs the HIP path through the C-ABI")


@pytest.fixture(scope="session")
def oracle_lib():
    """The oracle library, built with gcc if it is not there yet."""
    import oracle
    oracle._load()
    return oracle
