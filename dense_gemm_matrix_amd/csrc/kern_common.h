// kern_common.h -- device helpers shared by the GEMM kernels: vector types,
// buffer resources, the direct-to-LDS load, wait counts and the epilogue.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "dgemm_internal.h"

namespace dgemm {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

constexpr uint32_t BUF_WORD3 = 0x00020000u;  // raw buffer: 32-bit data format, no swizzle

// A raw buffer resource covering [base, base + bytes), the range rounded up to
// 16 bytes.  The buffer unit range-checks whole dwords, so a range ending in
// the middle of a dword (an odd count of 16-bit elements) would return the
// last element as zero.  Rounding up is safe: bases and row pitches are 16-byte
// aligned, so the extra bytes share a 16-byte chunk (hence a page) with the
// last element; they are masked (A's K tail) or feed only unstored outputs
// (B's columns past N).  bytes <= 0 gives an empty range.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const char* base, int64_t bytes) {
    const int64_t rounded = bytes > 0 ? (bytes + 15) & ~(int64_t)15 : 0;
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)rounded, (int)BUF_WORD3);
}

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, int voffset) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voffset, 0, 0);
}

// Reinterpret a 32-bit word as fp32.  The word is taken by value: clang's
// __builtin_bit_cast applied directly to an ext-vector element subscript
// (v[e]) reads element 0 whatever e is, so callers pass v[e] through here.
__device__ __forceinline__ float as_float(uint32_t w) { return __builtin_bit_cast(float, w); }

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// One direct-to-LDS 16-byte-per-lane buffer load: lane l's 16 bytes from
// rsrc + voffset land at LDS byte lds + 16 l.  Issued as inline assembly so that
// the compiler does not guard every later LDS read with a wait for ALL such
// loads (it cannot tell which LDS bytes they write); the kernel waits for them
// explicitly with s_waitcnt vmcnt before the barrier that publishes a stage.
// An LDS DMA needs one wait state after the SALU write of M0 that it reads
// (the compiler keeps one instruction between them for its own LDS DMA), hence
// the s_nop.
// M0 is reserved to the compiler, which warns about the clobber; nothing else
// in these kernels uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds, int voffset) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds), "v"(voffset), "s"(rsrc)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt immediate: wait until at most vm vector-memory and lgkm LDS/scalar
// operations of this wave are outstanding.
constexpr int waitcnt_imm(int vm, int lgkm) {
    return (vm & 0xf) | ((vm >> 4) << 14) | (0x7 << 4) | ((lgkm & 0xf) << 8);
}

template <int OUT>
__device__ __forceinline__ float load_c(const char* C, int64_t idx) {
    if (OUT == OUT_F32) return *reinterpret_cast<const float*>(C + idx * 4);
    if (OUT == OUT_BF16) return (float)*reinterpret_cast<const __bf16*>(C + idx * 2);
    return (float)*reinterpret_cast<const _Float16*>(C + idx * 2);
}

template <int OUT>
__device__ __forceinline__ void store_c(char* C, int64_t idx, float v) {
    if (OUT == OUT_F32) {
        *reinterpret_cast<float*>(C + idx * 4) = v;
    } else if (OUT == OUT_BF16) {
        *reinterpret_cast<__bf16*>(C + idx * 2) = (__bf16)v;      // round to nearest even
    } else {
        *reinterpret_cast<_Float16*>(C + idx * 2) = (_Float16)v;  // round to nearest even
    }
}

// The fused epilogue on one fp32 sum s: alpha * s + beta * C_old + bias, then
// the optional ReLU (a NaN passes through), in fp32, before the one rounding
// to C's format.
template <int OUT>
__device__ __forceinline__ float epilogue(float s, const char* C, int64_t idx, float bias,
                                          const EpiArgs& e) {
    float v = e.alpha * s;
    if (e.beta != 0.0f) v += e.beta * load_c<OUT>(C, idx);
    v += bias;
    if (e.relu && v < 0.0f) v = 0.0f;
    return v;
}

// Epilogue of the GEMM kernels.  32x32 accumulator layout: lane (g, li) holds
// column li and, in register r, row 8 * (r / 4) + 4 * g + r % 4.  Elements
// outside M x N are not stored; `full` (the whole macro-tile lies inside, a
// wave-uniform fact) takes a copy of the loop without the per-element tests,
// which would otherwise become one branch per store.
template <int OUT, int MI, int NJ, bool EPI, bool FULL>
__device__ __forceinline__ void store_tile_impl(const f32x16 (&acc)[MI][NJ], char* C, int M, int N,
                                                int ldc, int row0, int col0, int g, int li,
                                                const EpiArgs& e) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj) {
            const int col = col0 + nj * 32 + li;
            float bias = 0.0f;
            if (EPI && e.bias && (FULL || col < N)) bias = e.bias[col];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = row0 + mi * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                if (FULL || (row < M && col < N)) {
                    const int64_t idx = (int64_t)row * ldc + col;
                    float v = acc[mi][nj][r];
                    if constexpr (EPI) v = epilogue<OUT>(v, C, idx, bias, e);
                    store_c<OUT>(C, idx, v);
                }
            }
        }
    }
}

// Two fp32 values rounded to nearest even in C's 16-bit format, `lo` in the
// low half of the word.
template <int OUT>
__device__ __forceinline__ uint32_t pack16(float lo, float hi) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    const f32x2 v = {lo, hi};
    if constexpr (OUT == OUT_BF16)
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
    else
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

// DPP quad permutation [1, 0, 3, 2]: lane l reads lane l ^ 1.
constexpr int DPP_QUAD_XOR1 = 1 | (0 << 2) | (3 << 4) | (2 << 6);

__device__ __forceinline__ uint32_t swap_adjacent_lanes(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, DPP_QUAD_XOR1, 0xf, 0xf, false);
}

// Epilogue for 16-bit C on a tile that lies wholly inside C.  In the 32x32
// layout an even lane l and lane l + 1 hold columns c and c + 1; registers r
// and r + 1 (r even) hold rows R and R + 1.  Each lane rounds its two values
// into one word; one exchange between the two lanes then gives the even lane
// row R, columns c .. c + 1, and the odd lane row R + 1, the same columns: one
// 4-byte store where the per-element form needs two 2-byte ones, and each
// half-wave store writes two 64-byte row pieces instead of one.  The epilogue
// and the rounding act on each value before the exchange, so the stored values
// are those of store_tile_impl.  Needs every lane of the wave active.
template <int OUT, int MI, int NJ, bool EPI>
__device__ __forceinline__ void store_tile16_full(const f32x16 (&acc)[MI][NJ], char* C, int ldc,
                                                  int row0, int col0, int g, int li,
                                                  const EpiArgs& e) {
    const int odd = li & 1;
    // v_perm_b32 takes bytes 0-3 from its second source and 4-7 from its first:
    // the even lane keeps its low half (row R) and takes the neighbour's; the odd
    // lane takes the neighbour's high half (row R + 1) and keeps its own.
    const uint32_t sel = odd ? 0x03020706u : 0x05040100u;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj) {
            const int col = col0 + nj * 32 + li;
            float bias = 0.0f;
            if (EPI && e.bias) bias = e.bias[col];
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const int row = row0 + mi * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                float v0 = acc[mi][nj][r];
                float v1 = acc[mi][nj][r + 1];
                if constexpr (EPI) {
                    v0 = epilogue<OUT>(v0, C, (int64_t)row * ldc + col, bias, e);
                    v1 = epilogue<OUT>(v1, C, (int64_t)(row + 1) * ldc + col, bias, e);
                }
                const uint32_t p = pack16<OUT>(v0, v1);
                const uint32_t w = __builtin_amdgcn_perm(swap_adjacent_lanes(p), p, sel);
                const int64_t idx = (int64_t)(row + odd) * ldc + (col - odd);
                *reinterpret_cast<uint32_t*>(C + idx * 2) = w;
            }
        }
    }
}

template <int OUT, int MI, int NJ, bool EPI>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[MI][NJ], char* C, int M, int N,
                                           int ldc, int row0, int col0, int g, int li,
                                           const EpiArgs& e, bool full) {
    if (full) {
        if constexpr (OUT == OUT_F32)
            store_tile_impl<OUT, MI, NJ, EPI, true>(acc, C, M, N, ldc, row0, col0, g, li, e);
        else
            store_tile16_full<OUT, MI, NJ, EPI>(acc, C, ldc, row0, col0, g, li, e);
    } else {
        store_tile_impl<OUT, MI, NJ, EPI, false>(acc, C, M, N, ldc, row0, col0, g, li, e);
    }
}

}  // namespace dgemm
