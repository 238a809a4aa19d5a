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

With the fused epilogue E = act(alpha*C64 + beta*C_old + bias) the GPU scales
its fp32 sum, adds the two other terms in fp32 and rounds once.  The sum's error
becomes |alpha|*tol*S; the fp32 multiply and two adds (or fused multiply-adds)
add at most 2^-22 * T with T = |alpha*C64| + |beta*C_old| + |bias| (a generous
count of 4 roundings of 2^-24 each); ReLU is 1-Lipschitz and cannot enlarge an
error; rounding to the output adds u_out*|E|:

    |C_gpu - E| <= (|alpha|*tol*S + 2^-22 * T) * (1 + u_out) + u_out*|E| + sub_out
"""
import numpy as np

U_OUT = {"f32": 2.0 ** -24, "bf16": 2.0 ** -8, "f16": 2.0 ** -11}
SUB_OUT = {"f32": 2.0 ** -150, "bf16": 2.0 ** -134, "f16": 2.0 ** -25}
TOL_MFMA = 1e-4
TOL_SPLIT_BF16 = 2e-3


def bound(C64: np.ndarray, S: np.ndarray, tol: float, out: str) -> np.ndarray:
    u = U_OUT[out]
    return tol * S * (1.0 + u) + u * np.abs(C64) + SUB_OUT[out]


def bound_epilogue(E: np.ndarray, T: np.ndarray, S: np.ndarray, alpha: float, tol: float,
                   out: str) -> np.ndarray:
    u = U_OUT[out]
    pre = tol * abs(alpha) * S + 2.0 ** -22 * T
    return pre * (1.0 + u) + u * np.abs(E) + SUB_OUT[out]


def check(C_gpu: np.ndarray, C64: np.ndarray, S: np.ndarray, tol: float, out: str,
          C_round=None, b: np.ndarray = None) -> dict:
    """Elementwise check.  C_gpu is the GPU result already widened to float64.

    C64 is the reference value (for an epilogue, E) and b the bound (default:
    bound(C64, S, tol, out)).  Returns ok, n_bad, max_ratio (max error /
    bound), the first failing index, and, when C_round (the oracle's direct
    rounding, widened) is given, the fraction of elements equal to it.
    """
    C_gpu = np.asarray(C_gpu, dtype=np.float64)
    if C_gpu.shape != C64.shape:
        raise ValueError(f"shape {C_gpu.shape} != oracle {C64.shape}")
    if b is None:
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
