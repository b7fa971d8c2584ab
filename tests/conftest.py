import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU case")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


@pytest.fixture(scope="session")
def libpkv():
    """The built library (built in-tree first if nothing is built yet)."""
    from paged_kv_cache_physical_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from paged_kv_cache_physical_amd import build
        build.build()
    return _lib.lib()
