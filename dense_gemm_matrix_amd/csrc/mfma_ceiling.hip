// mfma_ceiling.hip -- the matrix-instruction ceiling the bf16 GEMM kernel is
// measured against.  Not part of the GEMM: a separate library
// (libmfma_ceiling.so) that only the benchmark loads.
//
// One workgroup of 4 waves per CU, one wave per SIMD, each wave running
// exactly the 256 x 256 GEMM kernel's matrix instructions: per loop
// iteration 4 chunk pairs x 16 v_mfma_f32_32x32x16_bf16 on 4 x 4 blocks of
// 32 x 32 fp32 accumulators (256 per lane), in the kernel's serpentine block
// order, each pair with its own operand register set.  The operands are
// loaded once from a buffer of bf16 values (the caller draws them from the
// GEMM workload's distribution) and then stay in registers: no global, LDS or
// operand-read traffic at all.  Under the board's power limit, the rate this
// reaches is what the GEMM's own matrix instructions could reach if moving
// operands cost nothing, so the GEMM's rate divided by it is the fraction of
// the attainable matrix-unit throughput the data movement leaves.

#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int KP = 4;   // chunk pairs per iteration (one 64-deep K step of the GEMM)
constexpr int MB = 4;   // 32 x 32 blocks per wave, each way

// ops: 4096 u32x4 per workgroup-sized slice (lane-linear): set kp, A block mi
// at [(kp * 8 + mi) * 256 + tid], B block nj at [(kp * 8 + 4 + nj) * 256 + tid].
__global__ __launch_bounds__(256) void mfma_ceiling_kernel(const u32x4* __restrict__ ops,
                                                           float* __restrict__ sink, int iters) {
    const int tid = (int)threadIdx.x;
    u32x4 a[KP][MB], b[KP][MB];
#pragma unroll
    for (int kp = 0; kp < KP; ++kp)
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            a[kp][i] = ops[(kp * 8 + i) * 256 + tid];
            b[kp][i] = ops[(kp * 8 + 4 + i) * 256 + tid];
        }
    f32x16 acc[MB][MB];
#pragma unroll
    for (int mi = 0; mi < MB; ++mi)
#pragma unroll
        for (int nj = 0; nj < MB; ++nj)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][nj][r] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int kp = 0; kp < KP; ++kp) {
#pragma unroll
            for (int i = 0; i < MB * MB; ++i) {
                const int mi = i / MB;
                const int nj = (mi & 1) ? MB - 1 - i % MB : i % MB;
                acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, a[kp][mi]), __builtin_bit_cast(bf16x8, b[kp][nj]),
                    acc[mi][nj], 0, 0, 0);
            }
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int mi = 0; mi < MB; ++mi)
#pragma unroll
        for (int nj = 0; nj < MB; ++nj)
#pragma unroll
            for (int r = 0; r < 16; ++r) s += acc[mi][nj][r];
    sink[blockIdx.x * 256 + tid] = s;
}

}  // namespace

extern "C" {

// Enqueues one launch of `grid` workgroups x `iters` iterations on `stream`.
// ops: device buffer of 4096 x 16 bytes of bf16 bit patterns; sink: device
// buffer of grid x 256 floats.  Each launch performs
// grid * 4 waves * iters * 64 * 32768 floating-point operations.
// Returns 0, or the HIP error code of the launch.
int mfma_ceiling_run(const void* ops, float* sink, int iters, int grid, void* stream) {
    hipLaunchKernelGGL(mfma_ceiling_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream,
                       (const u32x4*)ops, sink, iters);
    return (int)hipGetLastError();
}

}  // extern "C"
