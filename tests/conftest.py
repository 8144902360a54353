import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU case")


@pytest.fixture(scope="session")
def oracle_pool():
    """Worker processes for the fp64 oracle (one BLAS thread each), shared by the tests that
    compare every row of a full-size chunk or batch."""
    from oracle.parallel import OraclePool
    pool = OraclePool()
    yield pool
    pool.close()
