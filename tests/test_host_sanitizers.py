"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Builds lib/libfa_varlen_host_asan.so (validation, work lists and library memory compiled by g++
with -fsanitize=address,undefined; any UB report aborts) and runs the C-ABI and work-list CPU
tests against it in a child process with the ASan runtime preloaded.  A sanitizer report fails
the child, and so this test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    r = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(_runtime("libasan.so") is None, reason="no g++ AddressSanitizer runtime")
def test_abi_and_worklist_tests_pass_under_asan_and_ubsan():
    sys.path.insert(0, ROOT)
    from variable_length_flashattention_fa_amd.csrc import build
    lib = build.build_host_sanitized()
    env = dict(os.environ, FA_VARLEN_LIB=lib, LD_PRELOAD=_runtime("libasan.so"),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py"), os.path.join(ROOT, "tests", "test_worklist.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error:" not in tail, tail
    assert " passed" in r.stdout, tail
