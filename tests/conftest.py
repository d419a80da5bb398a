import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def orc():
    """The oracle the pins run against: the default build, or the build named
    by MOE_ORACLE_LIB (test_oracle_sanitized.py runs the pins on an
    ASan/UBSan build that way)."""
    import oracle

    path = os.environ.get("MOE_ORACLE_LIB")
    return oracle.Oracle(path) if path else oracle.default()
