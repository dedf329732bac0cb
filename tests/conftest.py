import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the C-ABI library)")
    # tests/test_host_sanitizers.py runs the allocator tests in a child process against the
    # sanitized host-only build of the allocator
    host = os.environ.get("PKV_HOST_LIBRARY")
    if host:
        import paged_kv_cache_284_amd as pkv
        pkv.use_host_library(host)
