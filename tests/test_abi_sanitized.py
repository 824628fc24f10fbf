"""The C ABI tests again, against a build whose host code (api.cpp: argument
validation, workspace layout, error strings) runs under AddressSanitizer and
UndefinedBehaviorSanitizer.  CPU only: every call in tests/test_abi.py is
refused or returns before any HIP call.  A sanitizer report aborts the child
process, which fails this test with the report in its message."""
import os
import subprocess
import sys

import pytest

from sparse_moe_transformer_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_under_asan_and_ubsan():
    rt = build.asan_runtime()
    if rt is None:
        pytest.skip("the compiler's AddressSanitizer runtime is not installed")
    lib = build.build_sanitized()
    env = dict(os.environ)
    env.update({"LD_PRELOAD": rt, "MOE_FFN_LIB": lib,
                "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-4000:] + r.stderr[-4000:])
    assert "passed" in r.stdout
