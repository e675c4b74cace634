"""The C ABI's host side under AddressSanitizer and UndefinedBehaviorSanitizer:
api.cpp is rebuilt with both (device code unchanged) and the whole ABI test
file runs against that build in a child process with the shared ASan runtime
preloaded. Any sanitizer report fails the test. CPU only."""
import os
import subprocess
import sys

import pytest

from long_context_decode_lowram_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_pass_under_host_sanitizers():
    try:
        B.hipcc()
        runtime = B.asan_runtime()
    except RuntimeError as exc:
        pytest.skip(f"no sanitizer toolchain: {exc}")
    if not all(os.path.exists(os.path.join(B.BUILD, os.path.splitext(s)[0] + ".o")) for s in B.SOURCES):
        B.build()
    lib = B.build_sanitized()
    env = dict(os.environ, LOWRAM_LIBRARY=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q",
                        "-p", "no:cacheprovider", "-m", "not gpu"], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out
