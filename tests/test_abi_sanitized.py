"""The CPU ABI checks (tests/test_abi.py) run again against a host-side
AddressSanitizer + UndefinedBehaviorSanitizer build of the C ABI's host code
(csrc/api.cpp: validation, overflow checks, alias checks, workspace layout),
in a child process with gcc's ASan runtime preloaded.  Any sanitizer report
aborts that process and fails this test.  No GPU is used."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _libasan():
    gcc = shutil.which("gcc")
    if not gcc:
        return None
    p = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(_libasan() is None or shutil.which("g++") is None, reason="gcc's ASan runtime not available")
def test_abi_checks_under_host_sanitizers():
    from second_order_ssm_amd import build as B

    lib = B.build_host_sanitized()
    env = dict(os.environ, LD_PRELOAD=_libasan(), TWOMAMBA_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-3000:]
    assert r.returncode == 0, out[-3000:]
    assert " passed" in r.stdout
