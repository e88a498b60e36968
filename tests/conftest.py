"""Shared pytest configuration.

Markers: ``gpu`` marks tests that need the MI355X (HIP) device; everything
else runs on the CPU.  The repository root is put on ``sys.path`` so the
tests can import ``oracle`` (test infrastructure) and the product package.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a HIP GPU (MI355X, gfx950)")


@pytest.fixture(scope="session")
def ora():
    import oracle
    oracle._load()
    return oracle
