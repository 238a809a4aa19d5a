"""Non-finite inputs through every path.

The pages fix nothing for NaN or infinite inputs; the reading taken is IEEE
propagation through the products and the sums.  Inputs are small integers,
so every finite output has one exact value, with one NaN in A (row i0) and one
+inf in B (column j1), the matching column of A holding non-zero integers.
Expected: row i0 all NaN (NaN times anything is NaN); column j1, other rows,
infinite with the sign of A[i][k1]; every other element equal to the oracle's
value for the same inputs with the two entries set to zero (after the one
rounding to a 16-bit C).  The 3 x bf16 path splits x into bf16(x) and
bf16(x - bf16(x)); for x = inf the second part is inf - inf = NaN, so there
column j1 is only required to be non-finite (the documented behaviour)."""
import numpy as np
import pytest
import torch

import dense_gemm_matrix_amd as dg
import oracle
from synth_inputs import to_storage
from tests.gpu_util import dev_matrix, gap_untouched, sentinel_c, to64

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("no_stream_k")]

ENTRY = {"f32": dg.gemm_f32, "f32x3": dg.gemm_f32_3xbf16, "bf16": dg.gemm_bf16, "f16": dg.gemm_f16}
COMBOS = [("f32", "f32"), ("f32x3", "f32"), ("bf16", "f32"), ("bf16", "bf16"), ("f16", "f32"),
          ("f16", "f16")]


def inputs(M, N, K, seed, i0, k0, k1, j1):
    """(A64, B64) with the non-finite entries, and (A0, B0) with them zeroed."""
    rng = np.random.default_rng(seed)
    A = rng.integers(-8, 9, size=(M, K)).astype(np.float64)
    B = rng.integers(-8, 9, size=(K, N)).astype(np.float64)
    A[:, k1] = rng.choice([-3.0, -1.0, 1.0, 2.0, 5.0], size=M)
    A0, B0 = A.copy(), B.copy()
    A0[i0, k0] = 0.0
    B0[k1, j1] = 0.0
    A[i0, k0] = np.nan
    B[k1, j1] = np.inf
    return A, B, A0, B0


def expected(dtype, out, A, A0, B0, i0, k1, j1):
    C64, _ = oracle.gemm(dtype, to_storage(A0, dtype), to_storage(B0, dtype))
    E = C64 if out == "f32" else oracle.widen(out, oracle.round_to(out, C64))
    E = E.copy()
    E[:, j1] = np.sign(A[:, k1]) * np.inf
    E[i0, :] = np.nan
    return E


def check(C, E, i0, j1, inf_column_exact=True):
    M, N = E.shape
    nan_row = np.zeros((M, N), dtype=bool)
    nan_row[i0, :] = True
    col = np.zeros((M, N), dtype=bool)
    col[:, j1] = True
    col &= ~nan_row
    rest = ~(nan_row | col)
    assert np.isnan(C[nan_row]).all(), "the NaN row did not stay NaN"
    if inf_column_exact:
        assert np.array_equal(C[col], E[col]), "the infinite column differs"
    else:
        assert not np.isfinite(C[col]).any(), "the infinite column has finite values"
    assert np.array_equal(C[rest], E[rest]), "finite outputs differ from the oracle"


@pytest.mark.parametrize("grid128", [False, True])
@pytest.mark.parametrize("path,out", COMBOS)
def test_nan_row_and_infinite_column(path, out, grid128):
    """Through the plain entry point (the planner's plan: slice-K at this size),
    and through gemm_ex with the 128 x 128 grid kernel forced."""
    M, N, K = 200, 136, 300          # ragged in every dimension; k1 in the K tail step
    i0, k0, k1, j1 = 5, 17, 290, 130
    dtype = "f32" if path == "f32x3" else path
    A, B, A0, B0 = inputs(M, N, K, 7100 + COMBOS.index((path, out)), i0, k0, k1, j1)
    Ad = dev_matrix(to_storage(A, dtype), dtype)
    Bd = dev_matrix(to_storage(B, dtype), dtype)
    Cd = sentinel_c(M, N, out)
    if grid128:
        dg.dgemm_set_plan_override(dg.DGEMM_PLAN_GRID, 128, 128, 1)
        try:
            assert dg.gemm_ex_plan(path, M, N, K, 0, out_same=(out != "f32"))["tile_rows"] == 128
            dg.gemm_ex(Ad, Bd, Cd, in_fmt="f32x3" if path == "f32x3" else None)
        finally:
            dg.dgemm_set_plan_override(dg.DGEMM_PLAN_AUTO)
    else:
        assert dg.gemm_ex_plan(path, M, N, K, 0, out_same=(out != "f32"))["tile_rows"] == 32
        ENTRY[path](Ad, Bd, Cd)
    torch.cuda.synchronize()
    print(f"nonfinite {path}->{out} {M}x{N}x{K} grid128={grid128}", flush=True)
    check(to64(Cd), expected(dtype, out, A, A0, B0, i0, k1, j1), i0, j1,
          inf_column_exact=(path != "f32x3"))
    assert gap_untouched(Cd)


@pytest.mark.parametrize("relu", [False, True])
def test_nonfinite_through_split_k_and_epilogue(relu):
    """A split-K plan: the NaN and the infinity sit in one split's partial sums and
    must survive the reduction; with ReLU, -inf becomes 0 and NaN passes."""
    M, N, K = 64, 72, 4104
    i0, k0, k1, j1 = 3, 4000, 100, 70
    plan = dg.gemm_ex_plan("bf16", M, N, K, 1 << 30, out_same=True)
    assert plan["splits"] > 1
    A, B, A0, B0 = inputs(M, N, K, 7200 + int(relu), i0, k0, k1, j1)
    Ad = dev_matrix(to_storage(A, "bf16"), "bf16")
    Bd = dev_matrix(to_storage(B, "bf16"), "bf16")
    C = dg.matmul(Ad, Bd, out_dtype=torch.bfloat16, relu=relu)
    torch.cuda.synchronize()
    print(f"nonfinite split-K relu={relu} plan {plan}", flush=True)
    C64, _ = oracle.gemm("bf16", to_storage(A0, "bf16"), to_storage(B0, "bf16"))
    if relu:
        C64 = np.maximum(C64, 0.0)
    E = oracle.widen("bf16", oracle.round_to("bf16", C64)).copy()
    E[:, j1] = np.sign(A[:, k1]) * np.inf
    if relu:
        E[:, j1] = np.where(A[:, k1] > 0, np.inf, 0.0)
    E[i0, :] = np.nan
    check(to64(C), E, i0, j1)
