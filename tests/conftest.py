import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def _ensure_built():
    """Build only what is missing; a present library is used as it is."""
    import oracle

    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()
    try:
        from adam_zs_shard_amd import _build
    except ImportError:  # product package not present yet
        return
    if not os.path.exists(_build.LIB_PATH):
        _build.build()


@pytest.fixture(scope="session", autouse=True)
def built_libraries():
    _ensure_built()
    yield
