import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # sanitizer runs (tests/sanitize/run_sanitizers.py) point the tests at
    # sanitizer builds of the oracle and of the library
    orc = os.environ.get("KVQ_TEST_ORACLE_LIB")
    if orc:
        import oracle
        oracle.LIB = orc
    kvq = os.environ.get("KVQ_TEST_LIBKVQ")
    if kvq:
        import quantized_kv_cache_fp8_amd as K
        K.LIB_PATH = kvq


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    import oracle
    if not os.path.exists(oracle.LIB) and not os.environ.get("KVQ_TEST_ORACLE_LIB"):
        oracle.build()
    yield
