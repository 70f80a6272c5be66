import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running parity case at full workload size")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


def pytest_sessionstart(session):
    # A planted oracle mistake, for tests/test_oracle_mutations.py only: that
    # test runs the oracle's CPU pins in a pytest process of its own with
    # ORACLE_MUTANT naming the mistake, and expects them to fail.
    name = os.environ.get("ORACLE_MUTANT")
    if name:
        import oracle_mutants
        oracle_mutants.apply(name)
