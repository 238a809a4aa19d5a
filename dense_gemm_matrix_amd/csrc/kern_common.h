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
// to C's format.  C_old is the element at byte address p.
template <int OUT>
__device__ __forceinline__ float epilogue_at(float s, const char* p, float bias, const EpiArgs& e) {
    float v = e.alpha * s;
    if (e.beta != 0.0f) v += e.beta * load_c<OUT>(p, 0);
    v += bias;
    if (e.relu && v < 0.0f) v = 0.0f;
    return v;
}

// The same for element idx of C.
template <int OUT>
__device__ __forceinline__ float epilogue(float s, const char* C, int64_t idx, float bias,
                                          const EpiArgs& e) {
    return epilogue_at<OUT>(s, C + idx * (OUT == OUT_F32 ? 4 : 2), bias, e);
}

// Epilogue of the GEMM kernels.  32x32 accumulator layout: lane (g, li) holds
// column li and, in register r, row 8 * (r / 4) + 4 * g + r % 4 of its block.
//
// Every tile takes one branch-free path: a buffer resource over C from the
// wave's corner (row0, col0) to the end of C's valid region, stores at 32-bit
// byte offsets = a per-lane part + a wave-uniform part.  Elements past the last
// row fall outside the resource's range, and lanes whose column is past N get
// an offset beyond any range (OOB_LANE): the buffer unit drops those stores
// (and returns zeros for those loads), so nothing outside M x N is written and
// no element needs a test.  Offsets stay below 2^31 because a 256-row panel of
// C is under 2 GiB (the ABI's precondition) and a range is at most 2^31 - 16
// bytes.
constexpr uint32_t OOB_LANE = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t c_rsrc(char* C, int M, int N, int ldc, int row0,
                                                         int col0, int es) {
    char* base = C + ((int64_t)row0 * ldc + col0) * es;
    int64_t rem = ((int64_t)(M - 1 - row0) * ldc + (N - col0)) * es;
    if (rem > 0x7ffffff0) rem = 0x7ffffff0;
    return make_rsrc(base, rem);
}

template <int OUT>
__device__ __forceinline__ float load_c_at(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (OUT == OUT_F32)
        return as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
    const uint32_t h = __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
    if constexpr (OUT == OUT_BF16) return as_float(h << 16);
    return (float)__builtin_bit_cast(_Float16, (unsigned short)h);
}

// The fused epilogue on one fp32 sum s read through the C resource.
template <int OUT>
__device__ __forceinline__ float epilogue_rs(float s, __amdgpu_buffer_rsrc_t r, uint32_t off,
                                             float bias, const EpiArgs& e) {
    float v = e.alpha * s;
    if (e.beta != 0.0f) v += e.beta * load_c_at<OUT>(r, off);
    v += bias;
    if (e.relu && v < 0.0f) v = 0.0f;
    return v;
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

// One store per element: fp32 C, or 16-bit C when a tile's column edge falls
// between the two columns of a lane pair (N odd).
template <int OUT, int MI, int NJ, bool EPI>
__device__ __forceinline__ void store_elems(const f32x16 (&acc)[MI][NJ], __amdgpu_buffer_rsrc_t r,
                                           int N, int ldc, int col0, int g, int li,
                                           const EpiArgs& e) {
    constexpr int ES = OUT == OUT_F32 ? 4 : 2;
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj) {
        const int col = col0 + nj * 32 + li;
        const uint32_t lane = col < N ? (uint32_t)((4 * g * ldc + nj * 32 + li) * ES) : OOB_LANE;
        float bias = 0.0f;
        if (EPI && e.bias && col < N) bias = e.bias[col];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const uint32_t off = lane + (uint32_t)((mi * 32 + 8 * (rr >> 2) + (rr & 3)) * ldc * ES);
                float v = acc[mi][nj][rr];
                if constexpr (EPI) v = epilogue_rs<OUT>(v, r, off, bias, e);
                if constexpr (OUT == OUT_F32) {
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, (int)off, 0, 0);
                } else {
                    const uint32_t p = pack16<OUT>(v, 0.0f);
                    __builtin_amdgcn_raw_buffer_store_b16((unsigned short)p, r, (int)off, 0, 0);
                }
            }
        }
    }
}

// 16-bit C with both columns of every lane pair inside or both outside: an
// even lane l and lane l + 1 hold columns c and c + 1, and registers r and
// r + 1 (r even) rows R and R + 1.  Each lane rounds its two values into one
// word; one exchange between the two lanes then gives the even lane row R,
// columns c .. c + 1, and the odd lane row R + 1, the same columns: one 4-byte
// store where the per-element form needs two 2-byte ones, and each half-wave
// store writes two 64-byte row pieces instead of one.  The epilogue and the
// rounding act on each value before the exchange, so the stored values are
// those of store_elems.  Needs every lane of the wave active.
template <int OUT, int MI, int NJ, bool EPI>
__device__ __forceinline__ void store_pairs16(const f32x16 (&acc)[MI][NJ], __amdgpu_buffer_rsrc_t r,
                                              int N, int ldc, int col0, int g, int li,
                                              const EpiArgs& e) {
    const int odd = li & 1;
    // v_perm_b32 takes bytes 0-3 from its second source and 4-7 from its first:
    // the even lane keeps its low half (row R) and takes the neighbour's; the odd
    // lane takes the neighbour's high half (row R + 1) and keeps its own.
    const uint32_t sel = odd ? 0x03020706u : 0x05040100u;
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj) {
        const int col = col0 + nj * 32 + li;
        const uint32_t own = col < N ? (uint32_t)((4 * g * ldc + nj * 32 + li) * 2) : OOB_LANE;
        const uint32_t word = col - odd < N ? (uint32_t)(((4 * g + odd) * ldc + nj * 32 + li - odd) * 2)
                                            : OOB_LANE;
        float bias = 0.0f;
        if (EPI && e.bias && col < N) bias = e.bias[col];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
            for (int rr = 0; rr < 16; rr += 2) {
                const uint32_t rows = (uint32_t)((mi * 32 + 8 * (rr >> 2) + (rr & 3)) * ldc * 2);
                float v0 = acc[mi][nj][rr];
                float v1 = acc[mi][nj][rr + 1];
                if constexpr (EPI) {
                    v0 = epilogue_rs<OUT>(v0, r, own + rows, bias, e);
                    v1 = epilogue_rs<OUT>(v1, r, own + rows + (uint32_t)(ldc * 2), bias, e);
                }
                const uint32_t p = pack16<OUT>(v0, v1);
                const uint32_t w = __builtin_amdgcn_perm(swap_adjacent_lanes(p), p, sel);
                __builtin_amdgcn_raw_buffer_store_b32(w, r, (int)(word + rows), 0, 0);
            }
        }
    }
}

// PAIRS (16-bit C): the launch's N is even, so no lane pair straddles the
// column edge and every tile takes store_pairs16; with N odd the kernel is
// instantiated with store_elems instead (deciding inside the kernel costs
// registers on every tile).
template <int OUT, int MI, int NJ, bool EPI, bool PAIRS>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[MI][NJ], char* C, int M, int N,
                                           int ldc, int row0, int col0, int g, int li,
                                           const EpiArgs& e) {
    if (row0 >= M || col0 >= N) return;  // this wave's part of the tile lies outside C
    constexpr int ES = OUT == OUT_F32 ? 4 : 2;
    const __amdgpu_buffer_rsrc_t r = c_rsrc(C, M, N, ldc, row0, col0, ES);
    if constexpr (OUT != OUT_F32 && PAIRS)
        store_pairs16<OUT, MI, NJ, EPI>(acc, r, N, ldc, col0, g, li, e);
    else
        store_elems<OUT, MI, NJ, EPI>(acc, r, N, ldc, col0, g, li, e);
}

}  // namespace dgemm
