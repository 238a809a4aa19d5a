"""Builds tests/c_client/gemm_client: plain C (gcc), linked against the HIP
runtime and the in-tree libdgemm.so (found at run time through an rpath)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "dense_gemm_matrix_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
BIN = os.path.join(HERE, "gemm_client")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(HERE, "gemm_client.c"), "-o", BIN + ".tmp",
           "-L", PKG, "-ldgemm", "-Wl,-rpath,$ORIGIN/../../dense_gemm_matrix_amd",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(BIN + ".tmp", BIN)
    return BIN


if __name__ == "__main__":
    build(verbose=True)
