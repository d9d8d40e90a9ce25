import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)

_ORACLE_POOL = None


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    # The oracle's worker pool is forked here, before test collection imports
    # the HIP library and before any test touches the GPU, so that the
    # workers hold no GPU state.
    global _ORACLE_POOL
    from oracle.pool import OraclePool
    _ORACLE_POOL = OraclePool()


def pytest_unconfigure(config):
    if _ORACLE_POOL is not None:
        _ORACLE_POOL.close()


@pytest.fixture(scope="session")
def oracle_pool():
    """Single-thread oracle workers (up to 16) for checking many queries."""
    return _ORACLE_POOL
