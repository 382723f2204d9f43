"""The host-side ABI checks (tests/test_abi.py) against a build whose host
code runs under AddressSanitizer and UndefinedBehaviorSanitizer: argument
validation, shape tables and error bookkeeping without memory errors or
undefined behaviour.  CPU only (no call in those checks reaches the GPU)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_under_host_sanitizers(tmp_path):
    try:
        from non_gemm_amd import build_sanitized
    except ImportError:
        pytest.skip("the sanitized build script is not part of this tree")
    lib = build_sanitized.build(str(tmp_path))
    env = dict(os.environ, LD_PRELOAD=build_sanitized.asan_runtime(), LS_MI355_TEST_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "tests/test_abi.py"],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out
