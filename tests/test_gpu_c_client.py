"""The C ABI from a plain C program (tests/c_client/gemm_client.c), with no
Python or torch in the process that calls the library: HIP runtime calls for
memory and a stream, include/dgemm.h for the product, padded row pitches, and
a check that the gap of every C row survives.  Inputs come from the seeded
generators as raw files; small integers make every output exact, so the
program's C must equal the oracle's bit for bit."""
import os
import subprocess

import numpy as np
import pytest

import oracle
from synth_inputs import pair

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_client", "gemm_client")

# (entry, C format, M, N, K, alpha, relu); "ex-" entries go through gemm_ex with
# the workspace gemm_ex_plan asks for.
CASES = [
    ("bf16", "f32", 300, 264, 520, None, None),
    ("bf16", "same", 257, 136, 200, None, None),
    ("f16", "same", 200, 136, 4104, None, None),
    ("f32", "f32", 200, 136, 300, None, None),
    ("f32x3", "f32", 130, 72, 100, None, None),
    ("ex-bf16", "same", 64, 72, 4104, 0.5, 1),     # a split-K plan with the epilogue
    ("ex-f32", "f32", 96, 64, 2048, 1.0, 0),       # a slice-K plan (no workspace)
    ("ex-f16", "f32", 300, 264, 520, 0.5, 1),
    ("bf16", "f32", 0, 64, 64, None, None),        # empty output: a no-op
    ("f16", "f32", 64, 72, 0, None, None),         # K = 0 writes zeros
]

STORE = {"f32": np.float32, "bf16": np.uint16, "f16": np.float16}


@pytest.mark.parametrize("entry,out,M,N,K,alpha,relu", CASES)
def test_c_program_matches_the_oracle(tmp_path, entry, out, M, N, K, alpha, relu):
    assert os.path.exists(BIN), "tests/c_client/gemm_client is missing: run build() first"
    fmt = entry[3:] if entry.startswith("ex-") else entry
    dtype = "f32" if fmt == "f32x3" else fmt
    cfmt = dtype if out == "same" else "f32"
    A, B = pair(M, N, K, "ints", dtype, seed=9100 + M + K)
    a, b, c = tmp_path / "a.bin", tmp_path / "b.bin", tmp_path / "c.bin"
    np.ascontiguousarray(A).tofile(a)
    np.ascontiguousarray(B).tofile(b)
    args = [BIN, entry, out, str(M), str(N), str(K), str(a), str(b), str(c)]
    if alpha is not None:
        args += [repr(alpha), str(relu)]
    print("c client:", " ".join(args[1:6]), flush=True)
    r = subprocess.run(args, capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, f"exit {r.returncode}: {r.stderr}"
    C = np.fromfile(c, dtype=STORE[cfmt]).reshape(M, N)
    C64 = np.zeros((M, N)) if M * N * K == 0 else oracle.gemm(dtype, A, B)[0]
    if alpha is not None:
        C64 = oracle.epilogue(C64, alpha, 0.0, None, None, bool(relu))[0]
    expect = oracle.widen(cfmt, oracle.round_to(cfmt, C64))
    assert np.array_equal(oracle.widen(cfmt, C), expect)
