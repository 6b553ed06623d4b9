"""Shared test set-up: markers, paths, and the two native libraries.

GPU tests are marked ``gpu``; everything else runs on a CPU-only machine.
The oracle library is compiled here when it is missing (gcc is available on
every machine these tests run on).  The HIP library is never compiled by the
tests: run ``python -c "import __graft_entry__ as g; g.build()"`` first.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD MI355X (gfx950) GPU and libarp.so")


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    from oracle import LIB_PATH
    if not os.path.exists(LIB_PATH):
        from oracle.build import build
        build()
    yield
