"""The pass/fail rule for comparing a GPU result with the oracle.  TEST INFRASTRUCTURE.

The nine-levels tutorial ("CUDA GEMM优化九重天", section 3.3 on checking
correctness) says never to compare floating-point GEMM results for equality and
to tie the threshold to the precision used.  The rule here scales the threshold
by S[i][j] = sum_k |a_ik * b_kj|, the quantity that bounds any summation order's
rounding error, and adds one rounding of the result to the output format:

    |C_gpu - C64| <= tol * S * (1 + u_out) + u_out * |C64| + sub_out

tol    : 1e-4 for paths that accumulate exact products in fp32 (bf16, fp16 and
         fp32 matrix instructions), 2e-3 for a split-bf16 fp32 path.
u_out  : unit roundoff of C's format (2^-24 fp32, 2^-8 bf16, 2^-11 fp16).
sub_out: half the subnormal spacing of C's format (rounding near zero is
         absolute, not relative).

Derivation: an fp32 accumulator s of exact products satisfies |s - C64| <= tol*S;
rounding s once to the output adds at most u_out*|s| <= u_out*(|C64| + tol*S),
plus sub_out if the result lands in the subnormal range.
NaN or Inf in C_gpu always fails (all workloads here are finite).
"""
import numpy as np

U_OUT = {"f32": 2.0 ** -24, "bf16": 2.0 ** -8, "f16": 2.0 ** -11}
SUB_OUT = {"f32": 2.0 ** -150, "bf16": 2.0 ** -134, "f16": 2.0 ** -25}
TOL_MFMA = 1e-4
TOL_SPLIT_BF16 = 2e-3


def bound(C64: np.ndarray, S: np.ndarray, tol: float, out: str) -> np.ndarray:
    u = U_OUT[out]
    return tol * S * (1.0 + u) + u * np.abs(C64) + SUB_OUT[out]


def check(C_gpu: np.ndarray, C64: np.ndarray, S: np.ndarray, tol: float, out: str,
          C_round=None) -> dict:
    """Elementwise check.  C_gpu is the GPU result already widened to float64.

    Returns ok, n_bad, max_ratio (max error / bound), the first failing index,
    and, when C_round (the oracle's direct rounding, widened) is given, the
    fraction of elements equal to it.
    """
    C_gpu = np.asarray(C_gpu, dtype=np.float64)
    if C_gpu.shape != C64.shape:
        raise ValueError(f"shape {C_gpu.shape} != oracle {C64.shape}")
    b = bound(C64, S, tol, out)
    err = np.abs(C_gpu - C64)
    finite = np.isfinite(C_gpu)
    bad = ~finite | ~(err <= b)
    ratio = np.where(finite, err / b, np.inf)
    res = {
        "ok": not bool(bad.any()),
        "n_bad": int(bad.sum()),
        "max_ratio": float(ratio.max()) if ratio.size else 0.0,
        "first_bad": tuple(int(i) for i in np.argwhere(bad)[0]) if bad.any() else None,
    }
    if C_round is not None:
        res["exact_frac"] = float(np.mean(C_gpu == np.asarray(C_round, dtype=np.float64))) \
            if C_gpu.size else 1.0
    return res
