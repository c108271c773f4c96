"""The oracle's pins under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU).

oracle.c is built with -fsanitize=address,undefined (gcc) and every pin of
tests/test_oracle.py runs against that build in a child process that
preloads gcc's libasan (a sanitized shared library needs its runtime loaded
first).  Any out-of-bounds access, use after free or undefined behaviour in
the oracle aborts the child, and the test fails with the sanitizer's report.
Leak checking is off: the Python interpreter itself holds memory at exit.
The same sanitized-build methodology (suites run clean under ASan and UBSan)
is the one of the sam3d.cpp experiment page "Narrow F32 tile follow-up",
section "Release timing".
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.timeout(600)
def test_pins_clean_under_sanitizers():
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    oracle.build(0, force=True, sanitize=True)
    env = dict(os.environ)
    env.update(ORACLE_SANITIZE="1", LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", "test_oracle.py"), "-k", "test_pin or threads"]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=580)
    report = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, report
    assert "ERROR: AddressSanitizer" not in report and "runtime error" not in report, report
    assert " passed" in r.stdout, report


_OOB_CHILD = """
import ctypes, numpy as np, oracle
lib = oracle._load()
Q = np.ones((2, 4), np.float32); C = np.ones((3, 4), np.float32)
qi = np.array([0], np.int64); cj = np.array([3], np.int64)   # one row past C's end
out = np.empty(1, np.float64)
p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
lib.orc_pair_values(p(Q), p(C), 4, 0, 1, p(qi), p(cj), p(out))
print("not caught")
"""


@pytest.mark.timeout(120)
def test_sanitized_build_catches_out_of_bounds_read():
    """Non-vacuity: an oracle call that reads one row past its candidate
    array (bypassing the Python wrapper's range check) aborts under the
    sanitized build with AddressSanitizer's report."""
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    oracle.build(0, force=False, sanitize=True)
    env = dict(os.environ)
    env.update(ORACLE_SANITIZE="1", LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0",
               PYTHONPATH=ROOT)
    r = subprocess.run([sys.executable, "-c", _OOB_CHILD], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=100)
    assert r.returncode != 0 and "not caught" not in r.stdout
    assert "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]
