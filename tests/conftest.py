import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


@pytest.fixture(scope="session")
def librrb():
    """The built library; builds it in-tree only if nothing is built yet."""
    from reduce_rank_buffers_amd import _lib
    if not (os.path.exists(_lib.LIB_PATH) and os.path.exists(_lib.LIB_FENCED_PATH)):
        from reduce_rank_buffers_amd import build
        build.build()
    return _lib.lib()
