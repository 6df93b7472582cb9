"""The library's host-side code (argument checks, dispatch, the native page
pool) under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU: the
host-sanitizer build (host pass only; the kernels are not sanitized) is
loaded in a child process that preloads clang's ASan runtime and reruns the
host ABI tests and the page-pool tests (random scripts against the oracle's
model) against it.  Any heap/stack overflow, use after free or undefined
behaviour aborts the child."""
import os
import subprocess
import sys

import pytest

from flashattention_paged_kv_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(not os.path.exists(build.HIPCC) or not build.asan_runtime(),
                    reason="hipcc or clang's ASan runtime not available")
def test_host_code_under_asan_and_ubsan():
    lib = build.build_sanitized(verbose=False)
    env = dict(os.environ)
    env.update(PAGEDATTN_LIB=lib, LD_PRELOAD=build.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        "tests/test_abi_host.py", "tests/test_page_pool_host.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
