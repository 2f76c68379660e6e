import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def pytest_sessionstart(session):
    """Build libpa.so if nothing is built yet (tests load what is built)."""
    from paged_kv_cache_398_amd import build

    if not os.path.exists(build.LIB_PATH):
        build.build()
