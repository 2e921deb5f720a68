"""The library's host code (argument validation of the C ABI, the host
spectral step of the calibration) under AddressSanitizer and UBSan: the
sanitized build (host sources instrumented, kernels as usual) runs the whole
C-ABI test file in a child process with the ASan runtime preloaded; any
sanitizer report fails it. No GPU is needed: those tests make no GPU call."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_suite_under_asan_and_ubsan():
    from token_level_sparse_amd import build
    if not os.path.exists(build.HIPCC):
        pytest.skip("hipcc not available")
    lib = build.build_sanitized()
    rt = build.sanitizer_runtime()
    assert os.path.exists(rt), rt
    env = dict(os.environ, JSSA_LIBRARY=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out
