// splitk.hip -- the reduction that finishes a split-K GEMM on gfx950.
//
// A split-K launch leaves `splits` fp32 partial products W[z] (each M x ldw,
// ldw a multiple of 4) in the caller's workspace; this kernel sums them in
// ascending z (so the result does not depend on timing), applies the fused
// epilogue and rounds once to C's format.  It is elementwise and bound by HBM:
// per output it reads 4 * splits bytes and writes one element (plus C_old
// when beta != 0), so each thread takes four consecutive columns of one row
// and moves 16-byte pieces.

#include "kern_common.h"

namespace dgemm {
namespace {

constexpr int RED_THREADS = 256;

template <int OUT, bool EPI>
__global__ __launch_bounds__(RED_THREADS) void splitk_reduce_kernel(
    const float* __restrict__ W, int splits, int64_t zstride, int ldw, char* __restrict__ C,
    int ldc, int M, int N, EpiArgs e) {
    const int nq = ldw >> 2;
    const int64_t t = (int64_t)blockIdx.x * RED_THREADS + threadIdx.x;
    if (t >= (int64_t)M * nq) return;
    const int row = (int)(t / nq);
    const int col0 = (int)(t - (int64_t)row * nq) * 4;
    if (col0 >= N) return;

    const float* p = W + (int64_t)row * ldw + col0;
    f32x4 s = *(const f32x4*)p;
    for (int z = 1; z < splits; ++z) s += *(const f32x4*)(p + z * zstride);

    const int64_t base = (int64_t)row * ldc + col0;
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[j] = s[j];
        if constexpr (EPI) {
            if (col0 + j < N) {
                const float bias = e.bias ? e.bias[col0 + j] : 0.0f;
                v[j] = epilogue<OUT>(v[j], C, base + j, bias, e);
            }
        }
    }
    if (col0 + 4 <= N) {
        // C's base and row pitch are 16-byte aligned and col0 is a multiple
        // of 4, so the four outputs form one aligned 16- or 8-byte piece.
        if constexpr (OUT == OUT_F32) {
            *(f32x4*)(C + base * 4) = f32x4{v[0], v[1], v[2], v[3]};
        } else {
            typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
            u16x4 h;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (OUT == OUT_BF16)
                    h[j] = __builtin_bit_cast(unsigned short, (__bf16)v[j]);
                else
                    h[j] = __builtin_bit_cast(unsigned short, (_Float16)v[j]);
            }
            *(u16x4*)(C + base * 2) = h;
        }
    } else {
        for (int j = 0; j < 4; ++j)
            if (col0 + j < N) store_c<OUT>(C, base + j, v[j]);
    }
}

template <int OUT, bool EPI>
hipError_t go(const float* W, int splits, int64_t zstride, int ldw, char* C, int ldc, int M, int N,
              const EpiArgs& e, hipStream_t stream) {
    const int64_t threads = (int64_t)M * (ldw / 4);
    const int64_t blocks = (threads + RED_THREADS - 1) / RED_THREADS;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    EpiArgs ea = e;
    void* args[] = {&W, &splits, &zstride, &ldw, &C, &ldc, &M, &N, &ea};
    return hipLaunchKernel((const void*)splitk_reduce_kernel<OUT, EPI>, dim3((unsigned)blocks),
                           dim3(RED_THREADS), args, 0, stream);
}

template <int OUT>
hipError_t by_epi(bool epi, const float* W, int splits, int64_t zstride, int ldw, char* C, int ldc,
                  int M, int N, const EpiArgs& e, hipStream_t stream) {
    return epi ? go<OUT, true>(W, splits, zstride, ldw, C, ldc, M, N, e, stream)
               : go<OUT, false>(W, splits, zstride, ldw, C, ldc, M, N, e, stream);
}

}  // namespace

hipError_t launch_splitk_reduce(const float* W, int splits, int64_t zstride, int ldw, char* C,
                                int ldc, int M, int N, int out, bool epi, const EpiArgs& e,
                                hipStream_t stream) {
    if (ldw % 4 != 0 || splits < 1) return hipErrorInvalidValue;
    if (out == OUT_F32) return by_epi<OUT_F32>(epi, W, splits, zstride, ldw, C, ldc, M, N, e, stream);
    if (out == OUT_BF16) return by_epi<OUT_BF16>(epi, W, splits, zstride, ldw, C, ldc, M, N, e, stream);
    if (out == OUT_F16) return by_epi<OUT_F16>(epi, W, splits, zstride, ldw, C, ldc, M, N, e, stream);
    return hipErrorInvalidValue;
}

}  // namespace dgemm
