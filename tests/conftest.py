"""Shared test setup: markers and import path.

`-m "not gpu"` runs the oracle pins, host logic and C-ABI export checks on any
machine; `-m gpu` runs the parity tests that call the HIP library.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a gfx950 GPU and the HIP library")


@pytest.fixture(scope="session")
def oracle():
    import oracle as _oracle

    return _oracle
