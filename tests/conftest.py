import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
for _p in (ROOT, os.path.dirname(os.path.abspath(__file__))):
    if _p not in sys.path:
        sys.path.insert(0, _p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running case")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle

    oracle._load()
    return oracle


def pytest_sessionstart(session):
    # Sanitizer runs (tests/test_sanitizers_cpu.py) point the tests at instrumented builds
    # of the library and the oracle through these variables; unset, the in-tree builds load.
    lib = os.environ.get("QMOE_TEST_LIBRARY")
    if lib:
        from quantized_mixture_experts_amd import binding
        binding.LIB_PATH = lib
    olib = os.environ.get("QMOE_TEST_ORACLE_LIBRARY")
    if olib:
        import oracle
        oracle._LIB_PATH = olib
