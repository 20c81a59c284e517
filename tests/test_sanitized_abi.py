"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

tests/sanitize/build_sanitized.py builds api.cpp with g++ -fsanitize=address,undefined (kernel
launchers stubbed out); the ABI test files then run in a child process against that library
(FATTN_LIB), with the sanitizer runtime preloaded into the interpreter. Any out-of-bounds access,
use after free or undefined behaviour in argument checking, planning or error reporting aborts
that run. Leak checking is off: the interpreter and torch keep allocations until exit.
"""

import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ABI_TESTS = ["tests/test_abi.py", "tests/test_abi_backward.py", "tests/test_abi_paged.py",
             "tests/test_abi_varlen.py", "tests/test_binding_buffers.py",
             "tests/test_zz_no_alloc.py"]


def _runtime(name):
    path = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("g++") is None or _runtime("libasan.so") is None,
                    reason="needs g++ with the AddressSanitizer runtime")
def test_abi_tests_pass_under_address_and_undefined_sanitizers(tmp_path):
    sys.path.insert(0, os.path.join(HERE, "sanitize"))
    try:
        import build_sanitized
    finally:
        sys.path.pop(0)
    lib = build_sanitized.build(str(tmp_path))
    env = dict(os.environ, FATTN_LIB=lib, LD_PRELOAD=_runtime("libasan.so"),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p",
                        "no:cacheprovider", *ABI_TESTS], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout
