import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


@pytest.fixture(scope="session", autouse=True)
def _built_library():
    """libgqa.so is built in-tree by __graft_entry__.build().  A checkout with
    nothing built gets it built here, once (hipcc cross-compiles for gfx950
    without a GPU); an existing build is used as it is."""
    lib = os.path.join(ROOT, "gqa_kv_cache_02_amd", "libgqa.so")
    if not os.path.exists(lib):
        from gqa_kv_cache_02_amd import build
        build.build()
