import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _order(item) -> int:
    """Correctness first: the parity suites, then bench.py end to end, then the
    allocation-free entry point's test files (test_zz_*)."""
    name = os.path.basename(str(item.fspath))
    if name.startswith("test_zz_"):
        return 2
    if name.startswith("test_bench"):
        return 1
    return 0


def pytest_collection_modifyitems(session, config, items):
    items.sort(key=_order)  # stable: file and definition order kept within each group
