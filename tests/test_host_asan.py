"""The library's host code under AddressSanitizer, on the CPU.

Builds libsawkv.so with the host compilation instrumented (the sanitizer flag
goes to the host side only; device code is built as usual) into a temporary
folder, then runs tests/test_abi.py against that build in a child process with
the sanitizer's runtime preloaded: every entry point's argument validation,
error text and size arithmetic runs instrumented. Skipped where hipcc or the
runtime is missing.
"""
import glob
import os
import subprocess
import sys

import pytest

from int4_kv_cache_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def test_abi_under_address_sanitizer(tmp_path):
    try:
        cc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not found")
    rt = asan_runtime()
    if rt is None:
        pytest.skip("AddressSanitizer runtime not found")
    lib = str(tmp_path / "libsawkv_asan.so")
    cmd = [cc] + B.flags() + ["-Xarch_host", "-fsanitize=address",
                              "-Xarch_host", "-fno-omit-frame-pointer"] + B.SRCS + ["-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, SAWKV_TEST_LIB=lib, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"),
                        "-q", "-p", "no:cacheprovider"],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    text = r.stdout + r.stderr
    assert "AddressSanitizer" not in text, text[-4000:]
    assert r.returncode == 0, text[-4000:]
    assert " passed" in text
