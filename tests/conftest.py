"""Shared pytest set-up.

Markers: ``gpu`` tests need an MI355X (they call the HIP library through its
C ABI); everything else runs on the CPU. The oracle library is built on
first use if it is missing; the HIP library is built only if nothing is
built yet (``__graft_entry__.build()`` rebuilds it unconditionally).
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD MI355X GPU (HIP library parity tests)")


@pytest.fixture(scope="session")
def oracle():
    import oracle as _oracle
    _oracle._load()
    return _oracle


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")
