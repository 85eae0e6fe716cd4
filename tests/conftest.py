import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def orc():
    import oracle
    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()
    oracle.set_threads(min(16, os.cpu_count() or 1))
    return oracle
