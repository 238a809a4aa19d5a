"""CPU oracle for C = A*B (row-major, fp64 accumulation).  TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import this
package.  It shares no code with the HIP path and never calls it.

The arithmetic lives in gemm_oracle.c (plain triple loop, exact fp64 widening,
ascending-k fp64 sums, direct round-to-nearest-even output rounding); this file
only marshals numpy arrays into it.  See gemm_oracle.c for the citations.

Storage conventions (the bytes the GPU receives):
  "f32"  -> numpy float32
  "bf16" -> numpy uint16 holding bf16 bit patterns
  "f16"  -> numpy float16
"""
import ctypes
import os

import numpy as np

from .epilogue import epilogue  # noqa: F401  (re-exported)
from .parity import U_OUT, bound, bound_epilogue, check  # noqa: F401  (re-exported)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_CODES = {"f32": 0, "bf16": 1, "f16": 2}
_STORAGE = {"f32": np.float32, "bf16": np.uint16, "f16": np.float16}
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from .build import build
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_widen.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_long]
        lib.oracle_round.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_long]
        lib.oracle_gemm_rows.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_long, ctypes.c_void_p, ctypes.c_long,
            ctypes.c_void_p, ctypes.c_long, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        for f in (lib.oracle_widen, lib.oracle_round, lib.oracle_gemm_rows):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    """Host threads the oracle uses: the CPUs this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _as_storage(dtype: str, x: np.ndarray) -> np.ndarray:
    want = _STORAGE[dtype]
    if x.dtype != want:
        raise TypeError(f"{dtype} storage must be {np.dtype(want).name}, got {x.dtype}")
    return x


def widen(dtype: str, x: np.ndarray) -> np.ndarray:
    """Exact widening of storage values to fp64."""
    x = np.ascontiguousarray(_as_storage(dtype, x))
    out = np.empty(x.shape, dtype=np.float64)
    rc = _load().oracle_widen(_CODES[dtype], x.ctypes.data, out.ctypes.data, x.size)
    if rc:
        raise RuntimeError(f"oracle_widen failed ({rc})")
    return out


def round_to(dtype: str, x64: np.ndarray) -> np.ndarray:
    """Direct round-to-nearest-even of fp64 values to the storage format."""
    x64 = np.ascontiguousarray(x64, dtype=np.float64)
    out = np.empty(x64.shape, dtype=_STORAGE[dtype])
    rc = _load().oracle_round(_CODES[dtype], x64.ctypes.data, out.ctypes.data, x64.size)
    if rc:
        raise RuntimeError(f"oracle_round failed ({rc})")
    return out


def gemm(dtype: str, A: np.ndarray, B: np.ndarray, rows=None, nthreads: int = None):
    """(C64, S) for the listed rows of C = A*B (all rows when rows is None).

    A: [M, K] storage array (row pitch = A.strides[0]); B: [K, N].  Inner strides
    must be one element.  Returns two float64 arrays of shape [len(rows), N].
    """
    A = _as_storage(dtype, A)
    B = _as_storage(dtype, B)
    if A.ndim != 2 or B.ndim != 2 or A.shape[1] != B.shape[0]:
        raise ValueError(f"shape mismatch {A.shape} x {B.shape}")
    es = A.itemsize
    for X in (A, B):
        if X.shape[0] > 0 and X.shape[1] > 1 and X.strides[1] != es:
            raise ValueError("inner stride must be one element")
        if X.strides[0] % es or X.strides[0] < 0:
            raise ValueError("row stride must be a non-negative multiple of the element size")
    M, K = A.shape
    N = B.shape[1]
    lda = max(A.strides[0] // es, K)
    ldb = max(B.strides[0] // es, N)
    if rows is None:
        rows = np.arange(M, dtype=np.int64)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
    C64 = np.empty((rows.size, N), dtype=np.float64)
    S = np.empty((rows.size, N), dtype=np.float64)
    if nthreads is None:
        nthreads = default_threads()
    rc = _load().oracle_gemm_rows(_CODES[dtype], M, N, K, A.ctypes.data, lda, B.ctypes.data, ldb,
                                  rows.ctypes.data, rows.size, C64.ctypes.data, S.ctypes.data,
                                  int(nthreads))
    if rc:
        raise RuntimeError(f"oracle_gemm_rows failed ({rc})")
    return C64, S
