"""The host-side argument validation of every entry point under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only): the library is rebuilt with host
instrumentation and tests/test_abi.py runs against it in a child process with the
sanitizer runtime preloaded. Any report (a bad read or write, a misaligned access,
an overflow, an invalid shift) stops that process, and the test fails with its
output."""
import os
import subprocess
import sys

import pytest

import sanitize_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_validation_under_asan_and_ubsan():
    rt = sanitize_build.asan_runtime()
    if rt is None:
        pytest.skip("no clang ASan runtime under /opt/rocm/llvm")
    lib = sanitize_build.build()
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, GDNRT_ABI_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    for mark in ("ERROR: AddressSanitizer", "runtime error:", "SUMMARY: UndefinedBehaviorSanitizer"):
        assert mark not in out, out[-4000:]
    assert " passed" in r.stdout
