"""The library's host code (argument checks, scratch layouts, launch dispatch) under AddressSanitizer and
UndefinedBehaviorSanitizer: the sanitized build (sanitizers on the host pass only) runs the ABI tests in a child
process with the sanitizer runtime preloaded; any report fails the test. CPU only: every call those tests make
returns before touching a GPU."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm*/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _sources_newer_than(lib):
    srcs = glob.glob(os.path.join(ROOT, "sparse_top_attention_amd", "csrc", "*")) + [os.path.join(ROOT, "include", "qsa.h")]
    return any(os.path.getmtime(s) > os.path.getmtime(lib) for s in srcs)


def test_abi_checks_under_address_and_ub_sanitizers():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no clang AddressSanitizer runtime in this image")
    from sparse_top_attention_amd import build as b
    if not os.path.exists(b.SAN_LIB) or _sources_newer_than(b.SAN_LIB):
        b.build(sanitize=True)
    env = dict(os.environ, LD_PRELOAD=rt, QSA_TEST_LIB=b.SAN_LIB,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    check = ("import ctypes, sys; assert hasattr(ctypes.CDLL(None), '__asan_init'), 'sanitizer runtime not loaded'; "
             "import pytest; sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-m', 'not gpu', "
             f"'{os.path.join(ROOT, 'tests', 'test_abi.py')}']))")
    r = subprocess.run([sys.executable, "-c", check], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-3000:]
    assert "passed" in r.stdout
