"""The C-ABI layer's host code (argument checks, workspace carving, size
queries, error text, profiler, runner set-up) under AddressSanitizer and
UndefinedBehaviorSanitizer: the library is rebuilt with both sanitizers on its
host code (build.py --sanitize; device code unchanged) and the ABI tests run
against that copy in a child process that preloads the compiler's ASan runtime.
Any sanitizer report fails the test (halt_on_error; UBSan without recovery).
CPU only: no call here reaches a kernel."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def sanitized_lib():
    sys.path.insert(0, os.path.join(ROOT, "mxfp4_block_scaled_e2m1_amd"))
    import build
    try:
        runtime = build.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    return build.build(jobs=8, sanitize=True), runtime


@pytest.mark.timeout(600)
def test_abi_under_asan_and_ubsan(sanitized_lib):
    lib, runtime = sanitized_lib
    env = dict(os.environ)
    env.update(LD_PRELOAD=runtime, MXFP4_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q", "-s",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=500)
    out = r.stdout + r.stderr
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
