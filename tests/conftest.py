import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")
    mutant = os.environ.get("QLIN_ORACLE_MUTANT_LIB")
    if mutant:
        # a copy of the oracle with one mistake planted on purpose
        # (test_oracle_mutants.py): every test loads it instead, and nothing
        # rebuilds over it
        import oracle
        oracle._LIB_PATH = mutant
        oracle._lib = None
        oracle.build = lambda force=False: mutant


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.build()
    return oracle
