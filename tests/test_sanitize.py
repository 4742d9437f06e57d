"""The host side of the library under AddressSanitizer and UndefinedBehaviorSanitizer:
libzha_asan.so (host code instrumented, device code as usual) loaded by a clang-built
C program that runs the C-ABI checks of test_c_abi.py, with leak detection on and any
report fatal. No GPU: the calls return before anything is enqueued."""

import glob
import os
import shutil
import subprocess

import pytest

from tree_indexed_sparse_amd import build as B

import test_c_abi as CABI

CLANG = "/opt/rocm/llvm/bin/clang"


def _runtime_dir():
    hits = glob.glob("/opt/rocm*/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return os.path.dirname(hits[0]) if hits else None


@pytest.mark.timeout(600)
def test_host_checks_under_asan_and_ubsan(tmp_path):
    rt = _runtime_dir()
    if not os.path.exists(CLANG) or rt is None or shutil.which(B.hipcc()) is None and \
            not os.path.exists(B.hipcc()):
        pytest.skip("clang, its ASan runtime or hipcc is missing")
    lib = B.build(sanitize=True)
    src = tmp_path / "main.c"
    src.write_text(CABI.PROGRAM)
    exe = tmp_path / "main"
    libdir = os.path.dirname(lib)
    cmd = [CLANG, "-std=c99", "-Wall", "-Werror", "-fsanitize=address,undefined", "-shared-libsan",
           "-fno-omit-frame-pointer", "-g", "-I", os.path.join(B.ROOT, "include"), str(src),
           "-o", str(exe), f"-L{libdir}", "-lzha_asan", f"-Wl,-rpath,{libdir}", f"-Wl,-rpath,{rt}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("OK")
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
