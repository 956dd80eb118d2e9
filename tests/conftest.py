import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    # the sanitizer run (tests/test_sanitized_host.py) loads a host-instrumented build
    lib = os.environ.get("GA_LIBRARY_UNDER_TEST")
    if lib:
        import paged_kv_cache_write_amd as ga
        ga.select_library(lib)
