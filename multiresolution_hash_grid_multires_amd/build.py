"""Build the HIP library ``libhashenc.so`` in-tree for gfx950 with hipcc.

Each source compiles to its own object (in parallel, under ``_build/`` at the repository
root), then hipcc links the shared library.  Run ``python -m
multiresolution_hash_grid_multires_amd.build`` (or call ``build_library()``).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ_DIR = os.path.join(ROOT, "_build", "hashenc")
LIB_PATH = os.path.join(PKG_DIR, "libhashenc.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++20",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # keep packed-fp32 instructions out of generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # hardware float atomics for unreturned fp32 adds (buffers are coarse-grained)
    "-munsafe-fp-atomics",
    "-fvisibility=hidden",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _jobs() -> int:
    try:
        n = int(os.environ.get("MAX_JOBS", "0"))
    except ValueError:
        n = 0
    return max(1, min(n or (os.cpu_count() or 1), 16))


def build_library(force: bool = True, verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(OBJ_DIR, exist_ok=True)
    flags = [*HIPCC_FLAGS, *(extra_flags or []), f"-I{INCLUDE}", f"-I{CSRC}"]

    def compile_one(src: str) -> str:
        obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
        cmd = [hipcc, *flags, "-c", "-o", obj, src]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        return obj

    with ThreadPoolExecutor(max_workers=_jobs()) as pool:
        objs = list(pool.map(compile_one, sources()))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose=True))
    sys.exit(0)
