"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU).

api.hip (every entry point's argument checks, workspace layouts and status
codes) is rebuilt with the sanitizers on its host side only (hipcc
-Xarch_host -fsanitize=...; the device code is not instrumented) and linked
with the library's other objects; the CPU tests that call the library
(tests/test_host.py, the host checks of the no-allocation entry point,
tests/test_no_fallback.py) then run against that build in a child process
that preloads clang's AddressSanitizer runtime.  Any out-of-bounds access or
undefined behaviour in the host code aborts the child and fails this test.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "farthest_vector_search_amd")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.timeout(900)
def test_host_code_clean_under_sanitizers(tmp_path):
    asan = _asan_runtime()
    if asan is None or not os.path.exists(HIPCC):
        pytest.skip("hipcc or clang's AddressSanitizer runtime is not installed")
    from farthest_vector_search_amd import build as b
    objs = [os.path.join(b.BUILD, os.path.splitext(s)[0] + ".o") for s in b.SOURCES if s != "api.hip"]
    if not all(os.path.exists(o) for o in objs):
        b.build(verbose=False)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer"]
    api_o = str(tmp_path / "api.o")
    lib = str(tmp_path / "libvs_san.so")
    flags = [f for f in b.FLAGS if f != "-O3"] + ["-O1", "-g"]
    r = subprocess.run([HIPCC, *flags, *san, "-c", os.path.join(b.CSRC, "api.hip"), "-o", api_o],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([HIPCC, f"--offload-arch={b.ARCH}", "-shared", "-fPIC", *san, "-o", lib,
                        api_o, *objs], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    child = (
        "import sys\n"
        f"sys.path.insert(0, {os.path.join(ROOT, 'tests')!r})\n"
        f"sys.path.insert(0, {ROOT!r})\n"
        "import farthest_vector_search_amd as vs\n"
        f"vs.LIB_PATH = {lib!r}\n"
        "import pytest\n"
        "sys.exit(pytest.main(['-q', '-x', '-m', 'not gpu', '-p', 'no:cacheprovider',\n"
        f"    {os.path.join(ROOT, 'tests', 'test_host.py')!r},\n"
        f"    {os.path.join(ROOT, 'tests', 'test_zz_no_alloc.py')!r},\n"
        f"    {os.path.join(ROOT, 'tests', 'test_no_fallback.py')!r}]))\n")
    env = dict(os.environ)
    env.update(LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-c", child], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout
