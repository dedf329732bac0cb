"""The host allocator under AddressSanitizer and UndefinedBehaviorSanitizer.

csrc/alloc.cpp (block allocator, copy-on-write forks, prefix cache, swap bookkeeping; plain
C++17 with no HIP) is built alone by the host compiler with -fsanitize=address,undefined and
-fno-sanitize-recover=all, and the allocator, prefix-cache and swap tests run against that build
in a child process with the ASan runtime preloaded.  Any invalid access, leak-free misuse or
undefined behaviour aborts the child, so the test passes only if the whole run is clean.
"""
import os
import subprocess
import sys

import pytest

from paged_kv_cache_284_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SUITES = ["tests/test_lib_allocator.py", "tests/test_lib_prefix_cache.py",
          "tests/test_lib_swap.py"]


def _asan_runtime() -> str:
    try:
        path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                              text=True, check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return ""
    return path if os.path.isabs(path) and os.path.exists(path) else ""


def test_allocator_suites_clean_under_asan_and_ubsan(tmp_path):
    runtime = _asan_runtime()
    if not runtime:
        pytest.skip("the host compiler has no ASan runtime")
    so = build.build_host_sanitized(str(tmp_path / "libpagedkv_host_asan.so"))
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": runtime,
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "PKV_HOST_LIBRARY": so,
        "HYPOTHESIS_PROFILE": env.get("HYPOTHESIS_PROFILE", "default"),
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", *SUITES], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, out
    assert " passed" in r.stdout, out
