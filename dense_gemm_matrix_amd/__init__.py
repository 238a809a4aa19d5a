"""Dense GEMM C = A*B for AMD MI355X (gfx950): hand-written HIP kernels behind a
C ABI (include/dgemm.h), with a thin ctypes binding of the same names."""
from ._binding import (  # noqa: F401
    DGEMM_ACT_NONE, DGEMM_ACT_RELU, DGEMM_ERR_ALIAS, DGEMM_ERR_DEVICE, DGEMM_ERR_INVALID_VALUE, DGEMM_ERR_LAUNCH,
    DGEMM_ERR_LEADING_DIM, DGEMM_ERR_MISALIGNED, DGEMM_ERR_SCRATCH_SIZE, DGEMM_ERR_TOO_LARGE,
    DGEMM_OK, DGEMM_STATIC_SCRATCH_BYTES,
    DGEMM_OUT_F32, DGEMM_OUT_SAME, DGEMM_PLAN_AUTO, DGEMM_PLAN_GRID, DGEMM_PLAN_STREAM_K,
    DGEMM_PLAN_NO_STREAM_K, LIB_PATH,
    DgemmError, dgemm_set_plan_override, dgemm_set_stream_k_wait_us, dgemm_status_string,
    dgemm_stream_k_schedule,
    dgemm_tile_map, gemm_bf16, gemm_ex, gemm_ex_plan, gemm_ex_static, gemm_f16, gemm_f32, gemm_f32_3xbf16,
    matmul, raw,
)
