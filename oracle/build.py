"""Builds liboracle.so from gemm_oracle.c with the host C compiler.

Test infrastructure: the oracle is compiled with -ffp-contract=off and without
fast-math, so every fp64 product and sum is rounded exactly as written.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gemm_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O3", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-pthread", "-std=c11", "-Wall", "-Wextra", SRC, "-o", LIB, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
