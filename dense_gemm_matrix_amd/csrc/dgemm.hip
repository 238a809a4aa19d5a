// dgemm.hip -- dense GEMM C = A*B for gfx950 (MI355X), behind the C ABI of
// include/dgemm.h.
//
// One kernel template serves fp32, bf16 and fp16 inputs.  Per workgroup:
//
//   * a 256 x 256 output macro-tile, 256 threads = 4 waves of 64 lanes in a
//     2 x 2 layout, each wave owning a 128 x 128 sub-tile held as 4 x 4
//     v_mfma 32x32 accumulator blocks (256 fp32 accumulators per lane, kept in
//     registers for the whole K loop);
//   * per K step, a 256 x 128-byte slab of A and of B staged in LDS (BK = 64
//     elements for 16-bit inputs, 32 for fp32), double buffered: the next
//     step's global loads are in flight while the current step computes, and
//     one barrier per step separates the LDS write of step k+1 from the reads
//     of step k;
//   * A is staged as it lies in memory (K-contiguous rows).  B is row-major
//     (N-contiguous), but a matrix instruction wants each lane's operand to run
//     along K, so each thread loads an 8-row block of B and transposes it in
//     registers before writing it to LDS as K-contiguous rows;
//   * LDS rows are 8 chunks of 16 bytes; chunk c of row r is stored at slot
//     c ^ phi(r).  Only chunk bits are permuted, so every 16-byte access stays
//     aligned (the principle of the sgemm tf32 page's section 3 swizzles and
//     the hgemm page's section 2), and phi is chosen for the access patterns
//     used here: the matrix-operand reads (8 lanes on 8 consecutive rows, same
//     chunk) and both staging writes (8 lanes on 8 chunks of one row);
//   * a bijective workgroup -> tile map that keeps each XCD's workgroups on a
//     compact block of tiles (the sgemm tf32 page's section 4 Grid Swizzling,
//     adapted to 8 XCDs with private L2s);
//   * buffer loads with per-step resource descriptors: rows past M (A) and K
//     (B) fall outside the descriptor's range and read as zero, the K tail of
//     A is masked to exact zeros, and the epilogue stores only inside M x N.
//     No host padding (the nine-levels tutorial's section 2.9 and 6.1 offer
//     padding or predication; predication is chosen).
//
// gfx950 has no xf32 matrix instruction, so fp32 inputs use full-precision
// v_mfma_f32_32x32x2_f32.  Matrix instructions' internal k order is not
// observable through the ABI: a lane group's operand chunk carries the same k
// indices for A and for B, so any permutation of k inside an instruction
// cancels.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>

#include "dgemm.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

enum InFmt { IN_F32 = 0, IN_BF16 = 1, IN_F16 = 2 };
enum OutFmt { OUT_F32 = 0, OUT_BF16 = 1, OUT_F16 = 2 };

constexpr int BM = 256;                       // macro-tile rows
constexpr int BN = 256;                       // macro-tile columns
constexpr int NTHREADS = 256;                 // 4 waves
constexpr int ROW_CHUNKS = 8;                 // 16-byte chunks per staged row (128 bytes of K)
constexpr int STAGE_CHUNKS = BM * ROW_CHUNKS; // one operand's stage: 2048 chunks = 32 KiB
constexpr int GROUP_M = 4;                    // tile rows per strip in the tile walk
constexpr int NUM_XCD = 8;                    // XCDs that workgroups are dealt across
constexpr uint32_t BUF_WORD3 = 0x00020000u;   // raw buffer: 32-bit data format, no swizzle
constexpr int64_t DESC_LIMIT = (int64_t)1 << 31;

template <int IN> struct InTraits;
template <> struct InTraits<IN_F32> { static constexpr int esize = 4, epc = 4, bk = 32; };
template <> struct InTraits<IN_BF16> { static constexpr int esize = 2, epc = 8, bk = 64; };
template <> struct InTraits<IN_F16> { static constexpr int esize = 2, epc = 8, bk = 64; };
// epc = elements per 16-byte chunk; bk = elements of K per step = ROW_CHUNKS * epc.

int in_esize(int in) { return in == IN_F32 ? 4 : 2; }
int in_bk(int in) { return in == IN_F32 ? 32 : 64; }

// Workgroup -> output tile.  Step 1: workgroups are dealt to XCDs in turn, so
// wg % 8 is its XCD; give XCD x the contiguous run of tile indices
// [start_x, start_x + count_x), runs sized as evenly as possible.  Step 2: walk
// tile indices in strips GROUP_M tile-rows high, column by column, so a run of
// ~32 tiles covers a compact block (4 x 8 at 4096 x 4096).  Both steps are
// bijections for any tile counts (the last strip may be shorter).
__host__ __device__ inline void map_tile(int wg, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int ntiles = tiles_m * tiles_n;
    const int x = wg % NUM_XCD;
    const int local = wg / NUM_XCD;
    const int q = ntiles / NUM_XCD;
    const int r = ntiles % NUM_XCD;
    const int t = (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + local;
    const int per_strip = GROUP_M * tiles_n;
    const int strip = t / per_strip;
    const int first_m = strip * GROUP_M;
    const int rows_in_strip = (tiles_m - first_m) < GROUP_M ? (tiles_m - first_m) : GROUP_M;
    const int rem = t - strip * per_strip;
    tm = first_m + rem % rows_in_strip;
    tn = rem / rows_in_strip;
}

// LDS slot of chunk c in staged row r.  With phi(r) = (r ^ (r >> 3)) & 7, the 8
// consecutive rows an operand read touches get 8 distinct slots, and so do the
// 8 aligned rows of any 16-row group with equal parity.
__device__ __forceinline__ int lds_index(int row, int chunk) {
    return row * ROW_CHUNKS + (chunk ^ ((row ^ (row >> 3)) & 7));
}

// A raw buffer resource covering [base, base + bytes), the range rounded up to
// 16 bytes.  The buffer unit range-checks whole dwords, so a range ending in
// the middle of a dword (an odd count of 16-bit elements) would return the
// last element as zero.  Rounding up is safe: bases and row pitches are 16-byte
// aligned, so the extra bytes share a 16-byte chunk (hence a page) with the
// last element; they are masked (A's K tail) or feed only unstored outputs
// (B's columns past N).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const char* base, int64_t bytes) {
    const int64_t rounded = (bytes + 15) & ~(int64_t)15;
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)rounded, (int)BUF_WORD3);
}

// Reinterpret a 32-bit word as fp32.  The word is taken by value: clang's
// __builtin_bit_cast applied directly to an ext-vector element subscript
// (v[e]) reads element 0 whatever e is, so callers pass v[e] through here.
__device__ __forceinline__ float as_float(uint32_t w) { return __builtin_bit_cast(float, w); }

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, int voffset) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voffset, 0, 0);
}

// Zero the elements of a chunk at and after `valid` (valid <= 0: all of them).
template <int EPC>
__device__ __forceinline__ u32x4 mask_tail(u32x4 v, int valid) {
    u32x4 out;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        uint32_t w = v[d];
        if (EPC == 4) {
            w = (d < valid) ? w : 0u;
        } else {
            const uint32_t lo = (2 * d < valid) ? 0x0000ffffu : 0u;
            const uint32_t hi = (2 * d + 1 < valid) ? 0xffff0000u : 0u;
            w &= (lo | hi);
        }
        out[d] = w;
    }
    return out;
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

template <int IN, int OUT>
__global__ __launch_bounds__(NTHREADS) void gemm_kernel(
    const char* __restrict__ A, const char* __restrict__ B, char* __restrict__ C,
    int M, int N, int K, int lda, int ldb, int ldc, int tiles_m, int tiles_n) {
    using T = InTraits<IN>;
    constexpr int ES = T::esize;
    constexpr int EPC = T::epc;
    constexpr int BK = T::bk;

    // [stage][operand: 0 = A, 1 = B][chunk]: 2 x 2 x 32 KiB.
    __shared__ u32x4 lds[2][2][STAGE_CHUNKS];

    int tm, tn;
    map_tile((int)blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int tid = (int)threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int m0 = tm * BM;
    const int n0 = tn * BN;
    const int rows_a = (M - m0) < BM ? (M - m0) : BM;
    const int cols_b = (N - n0) < BN ? (N - n0) : BN;
    const int nk = (K + BK - 1) / BK;
    const bool ragged_k = (K % BK) != 0;

    // A staging: thread -> chunk ac of rows ar0 + 32 i, i = 0..7.
    const int ac = tid & 7;
    const int ar0 = tid >> 3;
    // B staging: thread -> a block of 8 K-rows (kb) by one 16-byte column chunk (nb).
    constexpr int KB_COUNT = BK / 8;  // 8 (16-bit) or 4 (fp32)
    const int kb = tid % KB_COUNT;
    const int nb = tid / KB_COUNT;

    int voff_a[8], voff_b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        voff_a[i] = (ar0 + 32 * i) * lda * ES + ac * 16;
        voff_b[i] = (kb * 8 + i) * ldb * ES + nb * 16;
    }

    u32x4 ra[8], rb[8];

    auto load_step = [&](int kt, bool tail) {
        const int k0 = kt * BK;
        const char* abase = A + ((int64_t)m0 * lda + k0) * ES;
        const int64_t abytes = ((int64_t)(rows_a - 1) * lda + (K - k0)) * ES;
        const __amdgpu_buffer_rsrc_t rsa = make_rsrc(abase, abytes);
        const int rows_b = (K - k0) < BK ? (K - k0) : BK;
        const char* bbase = B + ((int64_t)k0 * ldb + n0) * ES;
        const int64_t bbytes = ((int64_t)(rows_b - 1) * ldb + cols_b) * ES;
        const __amdgpu_buffer_rsrc_t rsb = make_rsrc(bbase, bbytes);
#pragma unroll
        for (int i = 0; i < 8; ++i) ra[i] = load16(rsa, voff_a[i]);
#pragma unroll
        for (int i = 0; i < 8; ++i) rb[i] = load16(rsb, voff_b[i]);
        if (tail) {
            // Columns of A at or past K hold other data (row padding or the next
            // row); they must be exact zeros, since the matching B rows are.
            const int valid = K - k0 - ac * EPC;
#pragma unroll
            for (int i = 0; i < 8; ++i) ra[i] = mask_tail<EPC>(ra[i], valid);
        }
    };

    auto store_step = [&](int s) {
#pragma unroll
        for (int i = 0; i < 8; ++i) lds[s][0][lds_index(ar0 + 32 * i, ac)] = ra[i];
        if (EPC == 8) {
            // 8 K-rows x 8 columns of 16-bit values -> 8 columns x 8 K values.
#pragma unroll
            for (int cc = 0; cc < 8; ++cc) {
                const int d = cc >> 1;
                u32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t x = rb[2 * e][d];
                    const uint32_t y = rb[2 * e + 1][d];
                    v[e] = (cc & 1) ? ((x >> 16) | (y & 0xffff0000u))
                                    : ((x & 0x0000ffffu) | (y << 16));
                }
                lds[s][1][lds_index(nb * 8 + cc, kb)] = v;
            }
        } else {
            // 8 K-rows x 4 fp32 columns -> 4 columns x two chunks of 4 K values.
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    u32x4 v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = rb[4 * h + e][cc];
                    lds[s][1][lds_index(nb * 4 + cc, kb * 2 + h)] = v;
                }
            }
        }
    };

    const int wm = wave >> 1;
    const int wn = wave & 1;
    const int g = lane >> 5;   // lane group: which chunk of a chunk pair
    const int li = lane & 31;  // row of A / column of B within a 32-block

    f32x16 acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int nj = 0; nj < 4; ++nj)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][nj][r] = 0.0f;

    auto compute_step = [&](int s) {
#pragma unroll
        for (int kp = 0; kp < ROW_CHUNKS / 2; ++kp) {
            const int ch = 2 * kp + g;
            u32x4 a[4], b[4];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) a[mi] = lds[s][0][lds_index(wm * 128 + mi * 32 + li, ch)];
#pragma unroll
            for (int nj = 0; nj < 4; ++nj) b[nj] = lds[s][1][lds_index(wn * 128 + nj * 32 + li, ch)];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
                for (int nj = 0; nj < 4; ++nj) {
                    if (IN == IN_BF16) {
                        acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(bf16x8, a[mi]), __builtin_bit_cast(bf16x8, b[nj]),
                            acc[mi][nj], 0, 0, 0);
                    } else if (IN == IN_F16) {
                        acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                            __builtin_bit_cast(f16x8, a[mi]), __builtin_bit_cast(f16x8, b[nj]),
                            acc[mi][nj], 0, 0, 0);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                                as_float(a[mi][e]), as_float(b[nj][e]), acc[mi][nj], 0, 0, 0);
                    }
                }
            }
        }
    };

    if (nk > 0) {
        load_step(0, ragged_k && nk == 1);
        store_step(0);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            const bool more = kt + 1 < nk;
            if (more) load_step(kt + 1, ragged_k && kt + 2 == nk);
            compute_step(cur);
            if (more) store_step(cur ^ 1);
            __syncthreads();
        }
    }

    // Epilogue.  32x32 accumulator layout: lane (g, li) holds column li and,
    // in register r, row 8 * (r / 4) + 4 * g + r % 4.
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int nj = 0; nj < 4; ++nj) {
            const int col = n0 + wn * 128 + nj * 32 + li;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * 128 + mi * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                if (row < M && col < N) store_c<OUT>(C, (int64_t)row * ldc + col, acc[mi][nj][r]);
            }
        }
    }
}

// ---------------------------------------------------------------- host side

std::atomic<int> g_device_state[256];  // 0 unknown, 1 gfx950, 2 other

int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return DGEMM_ERR_DEVICE;
    int st = dev < 256 ? g_device_state[dev].load(std::memory_order_relaxed) : 0;
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return DGEMM_ERR_DEVICE;
        st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        if (dev < 256) g_device_state[dev].store(st, std::memory_order_relaxed);
    }
    return st == 1 ? DGEMM_OK : DGEMM_ERR_DEVICE;
}

bool ranges_overlap(uintptr_t a0, int64_t alen, uintptr_t b0, int64_t blen) {
    if (alen <= 0 || blen <= 0) return false;
    return a0 < b0 + (uintptr_t)blen && b0 < a0 + (uintptr_t)alen;
}

int validate(int M, int N, int K, const void* A, int lda, const void* B, int ldb, const void* C,
             int ldc, int in, int es_out, int64_t* ntiles_out) {
    const int es = in_esize(in);
    if (M < 0 || N < 0 || K < 0) return DGEMM_ERR_INVALID_VALUE;
    const bool writes = M > 0 && N > 0;
    const bool reads = writes && K > 0;
    if (writes && !C) return DGEMM_ERR_INVALID_VALUE;
    if (reads && (!A || !B)) return DGEMM_ERR_INVALID_VALUE;
    if (lda < (K > 1 ? K : 1) || ldb < (N > 1 ? N : 1) || ldc < (N > 1 ? N : 1))
        return DGEMM_ERR_LEADING_DIM;
    if (writes && (((uintptr_t)C & 15) || ((int64_t)ldc * es_out) % 16))
        return DGEMM_ERR_MISALIGNED;
    if (reads && (((uintptr_t)A & 15) || ((uintptr_t)B & 15) || ((int64_t)lda * es) % 16 ||
                  ((int64_t)ldb * es) % 16))
        return DGEMM_ERR_MISALIGNED;
    if (reads) {
        const int64_t alen = ((int64_t)(M - 1) * lda + K) * es;
        const int64_t blen = ((int64_t)(K - 1) * ldb + N) * es;
        const int64_t clen = ((int64_t)(M - 1) * ldc + N) * es_out;
        if (ranges_overlap((uintptr_t)C, clen, (uintptr_t)A, alen) ||
            ranges_overlap((uintptr_t)C, clen, (uintptr_t)B, blen))
            return DGEMM_ERR_ALIAS;
    }
    // Buffer descriptors address one 256-row panel of A and one K step of B
    // with 32-bit offsets.
    if ((int64_t)BM * lda * es >= DESC_LIMIT || (int64_t)in_bk(in) * ldb * es >= DESC_LIMIT)
        return DGEMM_ERR_TOO_LARGE;
    const int64_t tiles = ((int64_t)(M + BM - 1) / BM) * ((int64_t)(N + BN - 1) / BN);
    if (tiles > INT32_MAX) return DGEMM_ERR_TOO_LARGE;
    *ntiles_out = tiles;
    return DGEMM_OK;
}

template <int IN, int OUT>
int launch(int M, int N, int K, const void* A, int lda, const void* B, int ldb, void* C, int ldc,
           int64_t ntiles, void* stream) {
    int tiles_m = (M + BM - 1) / BM;
    int tiles_n = (N + BN - 1) / BN;
    const char* a = (const char*)A;
    const char* b = (const char*)B;
    char* c = (char*)C;
    void* args[] = {&a, &b, &c, &M, &N, &K, &lda, &ldb, &ldc, &tiles_m, &tiles_n};
    hipError_t e = hipLaunchKernel((const void*)gemm_kernel<IN, OUT>, dim3((unsigned)ntiles),
                                   dim3(NTHREADS), args, 0, (hipStream_t)stream);
    return e == hipSuccess ? DGEMM_OK : DGEMM_ERR_LAUNCH;
}

template <int IN>
int gemm_entry(int M, int N, int K, const void* A, int lda, const void* B, int ldb, void* C,
               int ldc, int out, void* stream) {
    if (out != DGEMM_OUT_F32 && out != DGEMM_OUT_SAME) return DGEMM_ERR_INVALID_VALUE;
    const int es_out = out == DGEMM_OUT_F32 ? 4 : in_esize(IN);
    int64_t ntiles = 0;
    int st = validate(M, N, K, A, lda, B, ldb, C, ldc, IN, es_out, &ntiles);
    if (st != DGEMM_OK) return st;
    if (M == 0 || N == 0) return DGEMM_OK;
    st = check_device();
    if (st != DGEMM_OK) return st;
    if (out == DGEMM_OUT_F32) return launch<IN, OUT_F32>(M, N, K, A, lda, B, ldb, C, ldc, ntiles, stream);
    if (IN == IN_BF16) return launch<IN_BF16, OUT_BF16>(M, N, K, A, lda, B, ldb, C, ldc, ntiles, stream);
    return launch<IN_F16, OUT_F16>(M, N, K, A, lda, B, ldb, C, ldc, ntiles, stream);
}

}  // namespace

extern "C" {

int gemm_f32(int M, int N, int K, const float* A, int lda, const float* B, int ldb, float* C,
             int ldc, void* stream) {
    return gemm_entry<IN_F32>(M, N, K, A, lda, B, ldb, C, ldc, DGEMM_OUT_F32, stream);
}

int gemm_bf16(int M, int N, int K, const void* A, int lda, const void* B, int ldb, void* C,
              int ldc, int out, void* stream) {
    return gemm_entry<IN_BF16>(M, N, K, A, lda, B, ldb, C, ldc, out, stream);
}

int gemm_f16(int M, int N, int K, const void* A, int lda, const void* B, int ldb, void* C,
             int ldc, int out, void* stream) {
    return gemm_entry<IN_F16>(M, N, K, A, lda, B, ldb, C, ldc, out, stream);
}

const char* dgemm_status_string(int status) {
    switch (status) {
    case DGEMM_OK: return "DGEMM_OK";
    case DGEMM_ERR_INVALID_VALUE: return "DGEMM_ERR_INVALID_VALUE: negative size, NULL pointer or bad out";
    case DGEMM_ERR_LEADING_DIM: return "DGEMM_ERR_LEADING_DIM: a leading dimension is below its row length";
    case DGEMM_ERR_MISALIGNED: return "DGEMM_ERR_MISALIGNED: a pointer or row pitch is not 16-byte aligned";
    case DGEMM_ERR_ALIAS: return "DGEMM_ERR_ALIAS: C overlaps A or B";
    case DGEMM_ERR_TOO_LARGE: return "DGEMM_ERR_TOO_LARGE: a panel exceeds the 32-bit buffer range";
    case DGEMM_ERR_DEVICE: return "DGEMM_ERR_DEVICE: no gfx950 device is current";
    case DGEMM_ERR_LAUNCH: return "DGEMM_ERR_LAUNCH: the kernel launch failed";
    default: return "DGEMM: unknown status";
    }
}

int dgemm_tile_map(int M, int N, int in, int wg, int* tile_rows, int* tile_cols, int* num_wg,
                   int* tile_m, int* tile_n) {
    if (M < 0 || N < 0 || (in != IN_F32 && in != IN_BF16 && in != IN_F16))
        return DGEMM_ERR_INVALID_VALUE;
    const int64_t tm_count = ((int64_t)M + BM - 1) / BM;
    const int64_t tn_count = ((int64_t)N + BN - 1) / BN;
    if (tm_count * tn_count > INT32_MAX) return DGEMM_ERR_TOO_LARGE;
    const int nwg = (int)(tm_count * tn_count);
    if (tile_rows) *tile_rows = BM;
    if (tile_cols) *tile_cols = BN;
    if (num_wg) *num_wg = nwg;
    if (wg >= 0 && wg < nwg) {
        int tm = 0, tn = 0;
        map_tile(wg, (int)tm_count, (int)tn_count, tm, tn);
        if (tile_m) *tile_m = tm;
        if (tile_n) *tile_n = tn;
    }
    return DGEMM_OK;
}

}  // extern "C"
