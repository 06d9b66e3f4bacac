"""Build ``libfp8w.so`` (gfx950) in-tree with hipcc.

    python -m fp8_block_scaled_02_amd.build

The library is the HIP sources under ``csrc/`` linked into one shared object
next to this file, with rocBLAS for the dense GEMM of the large-M route.
Only the ``fp8w_*`` symbols of ``include/fp8w.h`` are exported.  Packed-fp32 instructions are disabled for the whole build.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfp8w.so")
SOURCES = ["quantize.hip", "gemv.hip", "dequant.hip", "read_ceiling.hip", "gemm.cpp", "api.cpp"]
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Wall", "-Wextra", "-Werror", "-Wno-unused-command-line-argument",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: libfp8w needs ROCm to build")
    return path


def build(verbose: bool = False) -> str:
    """Compile every source and link ``libfp8w.so``; returns its path."""
    out_dir = os.path.join(ROOT, "_build")
    os.makedirs(out_dir, exist_ok=True)
    cc = hipcc()

    def compile_one(src: str) -> str:
        obj = os.path.join(out_dir, src + ".o")
        lang = [] if src.endswith(".hip") else ["-x", "hip"]
        cmd = [cc, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError(f"hipcc failed on {src}")
        return obj

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    rocm_lib = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(cc))), "lib")
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp,
           "-L", rocm_lib, "-lrocblas", "-Wl,-rpath," + rocm_lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link of libfp8w.so failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
