"""Shared test setup: repository root on sys.path, the `gpu` marker, and the built libraries."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def oracle_lib():
    """Path of the oracle library, built once per session if it is missing."""
    import oracle

    if not os.path.exists(oracle.lib_path()):
        oracle.build()
    return oracle.lib_path()
