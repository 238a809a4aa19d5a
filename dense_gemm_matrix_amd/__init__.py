"""Dense GEMM C = A*B for AMD MI355X (gfx950): hand-written HIP kernels behind a
C ABI (include/dgemm.h), with a thin ctypes binding of the same names."""
from ._binding import (  # noqa: F401
    DGEMM_ACT_NONE, DGEMM_ACT_RELU, DGEMM_ERR_ALIAS, DGEMM_ERR_DEVICE, DGEMM_ERR_INVALID_VALUE, DGEMM_ERR_LAUNCH,
    DGEMM_ERR_LEADING_DIM, DGEMM_ERR_MISALIGNED, DGEMM_ERR_SCRATCH_SIZE, DGEMM_ERR_TOO_LARGE,
    DGEMM_OK, DGEMM_STATIC_SCRATCH_BYTES,
    DGEMM_OUT_F32, DGEMM_OUT_SAME, LIB_PATH, DgemmError, dgemm_status_string,
    dgemm_tile_map, gemm_bf16, gemm_ex, gemm_ex_plan, gemm_ex_static, gemm_f16, gemm_f32, gemm_f32_3xbf16,
    matmul, raw,
)
