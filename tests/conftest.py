import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size parity case (minutes of CPU oracle work)")


@pytest.fixture
def golden():
    import json

    def load(name):
        with open(os.path.join(GOLDEN, name)) as f:
            return json.load(f)
    return load


def ensure_library():
    """Load the built HIP library; build it only when nothing is built."""
    from pagedattention_pkv_store_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from pagedattention_pkv_store_amd.build import build
        build()
    return _lib.lib()


@pytest.fixture(scope="session")
def pkv_lib():
    return ensure_library()
