"""Compile the gfx950 HIP library (libzha.so) in-tree with hipcc.

Each source is compiled to an object in parallel, then linked into one shared library
next to this file. Packed FP32 instructions are disabled for all device code.
"""

from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libzha.so")
OBJDIR = os.path.join(ROOT, "_build")

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE,
    "-I", CSRC,
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else (shutil.which("hipcc") or "hipcc")


def sources() -> list:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer (the device code is built as
# usual): each sanitizer flag applies to the host compilation only.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libzha.so; returns its path.
    sanitize=True builds libzha_asan.so instead, with the host code under ASan and UBSan
    (load it from a program built with clang's -fsanitize=address)."""
    objdir = OBJDIR + ("_asan" if sanitize else "")
    lib = LIB.replace("libzha.so", "libzha_asan.so") if sanitize else LIB
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()
    extra = HOST_SANITIZE if sanitize else []

    def compile_one(src: str) -> str:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [cc, *FLAGS, *extra, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, sources()))
    tmp = lib + ".tmp"
    link_extra = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-shared-libsan"] if sanitize else []
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    import sys

    print(build(verbose=True, sanitize="--sanitize" in sys.argv))
