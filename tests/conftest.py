"""Shared fixtures and markers.

``gpu`` tests need an MI355X and the built ``libfp8w.so``; everything else
runs on a CPU-only host.  The oracle under ``oracle/`` is test infrastructure
and is imported only from tests, the smoke check and the benchmark's CPU leg.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and libfp8w.so")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle.build(force=False)
    return oracle
