"""Builds libdgemm.so (the HIP kernels and the C ABI of include/dgemm.h) for gfx950.

The library is built in-tree so that it travels with the source tree.
"""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
# the C ABI and planner, then one file per kernel family
SOURCES = [os.path.join(CSRC, f)
           for f in ("dgemm.hip", "gemm16.hip", "gemm32.hip", "slicek16.hip", "splitk.hip")]
LIB = os.path.join(PKG, "libdgemm.so")
# The benchmark's matrix-instruction ceiling kernel: a library of its own,
# loaded only by bench.py, never by the package.
CEILING_SRC = os.path.join(CSRC, "mfma_ceiling.hip")
CEILING_LIB = os.path.join(PKG, "libmfma_ceiling.so")
OBJ_DIR = os.path.join(PKG, "_build")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the kernels' main loops are fully unrolled schedules; let #pragma unroll
    # expand the 3 x bf16 kernel's (larger than the default limit allows)
    "-mllvm", "-pragma-unroll-threshold=65536",
    "-Wall",
]


def build(verbose: bool = False) -> str:
    """Compiles every source to an object (in parallel), then links the library."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(OBJ_DIR, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include")]

    def compile_one(src):
        obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
        cmd = [hipcc, *HIPCC_FLAGS, "-c", *inc, src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as pool:
        objs = list(pool.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    tmp = CEILING_LIB + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-shared", CEILING_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, CEILING_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
