"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU): littlebit_host.hip is rebuilt with the sanitizers, linked with the
regular device objects, and tests/test_abi.py runs against that library in a
child process with the sanitizer runtime preloaded.  Any report halts the
child, so the test fails on the first finding."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_pass_under_host_sanitizers():
    from binary_rank_gemv_amd import build
    if not os.path.exists(os.path.join(build.OBJDIR, "decode.hip.o")):
        pytest.skip("library objects not built (python -m binary_rank_gemv_amd.build)")
    runtime = build.asan_runtime()
    if not runtime:
        pytest.skip("no AddressSanitizer runtime found")
    lib = build.build_sanitized_host()
    env = dict(os.environ, LITTLEBIT_LIBRARY=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    p = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       env=env, capture_output=True, text=True, timeout=600, cwd=ROOT)
    out = p.stdout + p.stderr
    assert p.returncode == 0 and "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert " passed" in out
