"""The fused epilogue, in fp64.  TEST INFRASTRUCTURE.

    E[i][j] = act(alpha * C64[i][j] + beta * C_old[i][j] + bias[j])

The hgemm page ("[CUDA 优化实战] hgemm - 超越 cuBLAS", closing discussion) names
the library kernel it races, a bf16 tensor-core GEMM with a ReLU fused into its
epilogue; the pages' own kernels have no epilogue beyond the output conversion.
The scaling by alpha and beta and the per-column bias are the conventional
companions of such an epilogue (BLAS's C := alpha*A*B + beta*C; a bias per output
column as in a linear layer); that reading, and ReLU as act(x) = 0 for x < 0
and x otherwise (a NaN passes through), is this oracle's definition.

Every operation is one fp64 operation on exactly widened values, so with the
dyadic inputs the tests use the result is exact; the rounding to the output
format happens afterwards, once (oracle.round_to).  C_old is only read when
beta != 0, so a NaN there is not propagated by a zero beta.
"""
import numpy as np


def epilogue(C64: np.ndarray, alpha: float, beta: float = 0.0, C_old64: np.ndarray = None,
             bias64: np.ndarray = None, relu: bool = False):
    """Returns (E, T): the epilogue's exact-input result and the magnitude sum
    T = |alpha * C64| + |beta * C_old| + |bias| that bounds its rounding."""
    C64 = np.asarray(C64, dtype=np.float64)
    v = float(alpha) * C64
    T = np.abs(v)
    if beta != 0.0:
        if C_old64 is None or np.shape(C_old64) != C64.shape:
            raise ValueError("beta != 0 needs C_old of C's shape")
        w = float(beta) * np.asarray(C_old64, dtype=np.float64)
        v = v + w
        T = T + np.abs(w)
    if bias64 is not None:
        b = np.asarray(bias64, dtype=np.float64).reshape(1, -1)
        if b.shape[1] != C64.shape[1]:
            raise ValueError("bias needs one value per column")
        v = v + b
        T = T + np.abs(b)
    if relu:
        v = np.where(v < 0.0, 0.0, v)
    return v, T
