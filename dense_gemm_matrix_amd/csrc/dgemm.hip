// dgemm.hip -- dense GEMM C = A*B for gfx950 (MI355X), behind the C ABI of
// include/dgemm.h.
//
// Two kernels share the tile map, the 256 x 256 macro-tile, the wave layout
// and the epilogue:
//
//   * gemm16_kernel (bf16 / fp16 inputs).  Both operands go global -> LDS with
//     direct-to-LDS buffer loads (no VGPR staging, no LDS write instructions)
//     into a ring of S16 stages of BK16-deep slabs (2 x 64 at present: of the
//     settings that fit 160 KiB, measured fastest; 4 x 32 and 5 x 32 were
//     slower), each issued one step before its use.  A is stored K-contiguous and read with ds_read_b128.  B is
//     stored as it lies in memory (row-major, N-contiguous) and read with
//     ds_read_b64_tr_b16: within each 16-lane group that instruction performs
//     a 4 x 4 transpose of 4-element row pieces, which hands every lane the
//     four consecutive k of one column that the matrix instruction's B operand
//     needs.  v_mfma_f32_32x32x16_{bf16,f16}.
//   * gemm_kernel (fp32 inputs).  gfx950 has no xf32 matrix instruction, so
//     products use full-precision v_mfma_f32_32x32x2_f32.  Operands are staged
//     through registers (B's 8 x 4 fp32 blocks are transposed by register
//     renaming), double-buffered in LDS with BK = 32.
//
// Shared structure, per workgroup: 256 threads = 4 waves of 64 lanes in a
// 2 x 2 layout, each wave owning a 128 x 128 sub-tile held as 4 x 4 blocks of
// 32 x 32 accumulators (256 fp32 per lane, register-resident for the whole K
// loop).  LDS rows are split into 16-byte chunks whose positions are XORed
// with a function of the row, so every 16-byte access stays aligned (the
// principle of the sgemm tf32 page's section 3 swizzles and the hgemm page's
// section 2) while the access patterns used here hit distinct LDS banks.  A
// bijective workgroup -> tile map keeps each XCD's workgroups on a compact
// block of tiles (the sgemm tf32 page's section 4 Grid Swizzling, adapted to 8
// XCDs with private L2s).  Buffer loads use per-step resource descriptors:
// rows past M (A) and past K (B) fall outside the range and read as zero, A's
// K tail is forced to exact zeros, and the epilogue stores only inside M x N;
// no host padding (the nine-levels tutorial's sections 2.9 and 6.1 offer
// padding or predication; predication is chosen).
//
// Matrix instructions' internal k order is not observable through the ABI: a
// lane group's operand carries the same k indices for A and for B, so any
// permutation of k inside an instruction cancels.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <type_traits>

#include "dgemm.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

enum InFmt { IN_F32 = 0, IN_BF16 = 1, IN_F16 = 2, IN_F32X3 = 3 };  // F32X3: fp32 via 3 x bf16
enum OutFmt { OUT_F32 = 0, OUT_BF16 = 1, OUT_F16 = 2 };

constexpr int BM = 256;                       // macro-tile rows
constexpr int BN = 256;                       // macro-tile columns
constexpr int NTHREADS = 256;                 // 4 waves
constexpr int GROUP_M = 4;                    // tile rows per strip in the tile walk
constexpr int NUM_XCD = 8;                    // XCDs that workgroups are dealt across
constexpr uint32_t BUF_WORD3 = 0x00020000u;   // raw buffer: 32-bit data format, no swizzle
constexpr int64_t DESC_LIMIT = (int64_t)1 << 31;

// K per step: 32 for both kernels (fp32: 128-byte LDS rows; 16-bit: 64-byte rows).
constexpr int BK = 32;

int in_esize(int in) { return (in == IN_F32 || in == IN_F32X3) ? 4 : 2; }

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
__device__ __forceinline__ void store_c(char* C, int64_t idx, float v) {
    if (OUT == OUT_F32) {
        *reinterpret_cast<float*>(C + idx * 4) = v;
    } else if (OUT == OUT_BF16) {
        *reinterpret_cast<__bf16*>(C + idx * 2) = (__bf16)v;      // round to nearest even
    } else {
        *reinterpret_cast<_Float16*>(C + idx * 2) = (_Float16)v;  // round to nearest even
    }
}

// Epilogue shared by both kernels.  32x32 accumulator layout: lane (g, li)
// holds column li and, in register r, row 8 * (r / 4) + 4 * g + r % 4.
template <int OUT, int MI = 4, int NJ = 4>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[MI][NJ], char* C, int M, int N,
                                           int ldc, int row0, int col0, int g, int li) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj) {
            const int col = col0 + nj * 32 + li;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = row0 + mi * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                if (row < M && col < N) store_c<OUT>(C, (int64_t)row * ldc + col, acc[mi][nj][r]);
            }
        }
    }
}

// ---------------------------------------------------------------- 16-bit kernel

constexpr int BK16 = 64;                       // K per stage
constexpr int S16 = 2;                         // LDS stages
constexpr int KP16 = BK16 / 16;                // 16-k chunk pairs per stage
constexpr int A16_CH = BK16 / 8;               // 16-byte chunks per A row
constexpr int A16_ROW = BK16 * 2;              // bytes per staged A row
constexpr int A16_RPB = 1024 / A16_ROW;        // A rows per 1 KiB load block

// Macro-tile TBM x TBN, 4 waves in a 2 x 2 layout, each wave (TBM/2) x (TBN/2)
// = MI x NJ blocks of 32 x 32 accumulators.
template <int TBM, int TBN>
struct Tile16 {
    static constexpr int MI = TBM / 64;
    static constexpr int NJ = TBN / 64;
    static constexpr int A_STAGE = TBM * A16_ROW;        // bytes per A stage
    static constexpr int B_ROW = TBN * 2;                // bytes per staged B row
    static constexpr int B_CH = TBN / 8;                 // 16-byte chunks per B row
    static constexpr int B_STAGE = BK16 * B_ROW;         // bytes per B stage
    static constexpr int B_RPB = 1024 / B_ROW;           // B rows per 1 KiB load block
    static constexpr int A_DMA = A_STAGE / 1024 / 4;     // direct-to-LDS loads per wave per stage
    static constexpr int B_DMA = B_STAGE / 1024 / 4;
    static constexpr int LOADS = A_DMA + B_DMA;
    static constexpr int NREAD = MI + 2 * NJ;            // fragment reads per chunk pair
    static constexpr int NMFMA = MI * NJ;                // MFMAs per chunk pair
    static_assert(TBM % 64 == 0 && TBN % 64 == 0 && TBM <= NTHREADS, "tile shape");
    static_assert(A_STAGE % 4096 == 0 && B_STAGE % 4096 == 0, "whole load blocks per wave");
    static_assert(S16 * (A_STAGE + B_STAGE) <= 160 * 1024, "LDS budget");
    static_assert((S16 - 1) * LOADS <= 63, "vmcnt range");
};

// Byte offset of chunk c (0..7) of A row r in a stage.  ds_read_b128 serves
// groups of 4 consecutive lanes from a 64-byte window of banks (measured on
// gfx950 with SQ_LDS_BANK_CONFLICT), and the 4 lanes of a group read 4
// consecutive rows at one chunk: a16_phi gives those rows 4 distinct slots.
__device__ __forceinline__ int a16_phi(int row) { return (row ^ (row >> 2)) & (A16_CH - 1); }
__device__ __forceinline__ int a16_off(int row, int chunk) {
    return row * A16_ROW + ((chunk ^ a16_phi(row)) << 4);
}
// Byte offset of chunk c of B row k in a stage with row pitch `row_bytes` (a
// multiple of 256).  ds_read_b64_tr_b16 serves 32 lanes from a 256-byte
// window (measured), and those 32 lanes read 4 consecutive k rows x 64 bytes;
// the XOR puts the four rows' pieces in distinct quarters of the window.
__device__ __forceinline__ int b16_swz(int k) { return ((k & 3) << 1) ^ ((k & 1) << 3); }
__device__ __forceinline__ int b16_off(int k, int chunk, int row_bytes) {
    return k * row_bytes + ((chunk ^ b16_swz(k)) << 4);
}

template <int IN, int OUT, int TBM, int TBN>
__global__ __launch_bounds__(NTHREADS) void gemm16_kernel(
    const char* __restrict__ A, const char* __restrict__ B, char* __restrict__ C,
    int M, int N, int K, int lda, int ldb, int ldc, int tiles_m, int tiles_n) {
    using T = Tile16<TBM, TBN>;
    constexpr int MI = T::MI, NJ = T::NJ;
    __shared__ __attribute__((aligned(1024))) char smem[S16 * (T::A_STAGE + T::B_STAGE)];
    char* const smA = smem;
    char* const smB = smem + S16 * T::A_STAGE;

    int tm, tn;
    map_tile((int)blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int tid = (int)threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in an SGPR
    const int m0 = tm * TBM;
    const int n0 = tn * TBN;
    const int rows_a = (M - m0) < TBM ? (M - m0) : TBM;
    const int cols_b = (N - n0) < TBN ? (N - n0) : TBN;
    const int nk = (K + BK16 - 1) / BK16;

    // Each direct-to-LDS instruction fills a 1 KiB block lane-linearly (lane l
    // -> bytes 16 l .. 16 l + 15), so the swizzle is applied on the global side:
    // lane l fetches the chunk that belongs in its slot.  Wave w fills the
    // blocks w * DMA .. (w + 1) * DMA - 1 of each operand's stage: for A,
    // A16_RPB rows of A16_CH chunks each; for B, B_RPB k-rows of B_CH chunks.
    int voffA[T::A_DMA], voffB[T::B_DMA];
#pragma unroll
    for (int j = 0; j < T::A_DMA; ++j) {
        const int rowA = (wave * T::A_DMA + j) * A16_RPB + lane / A16_CH;
        const int cA = (lane % A16_CH) ^ a16_phi(rowA);
        voffA[j] = rowA * lda * 2 + cA * 16;
    }
#pragma unroll
    for (int j = 0; j < T::B_DMA; ++j) {
        const int kB = (wave * T::B_DMA + j) * T::B_RPB + lane / T::B_CH;
        const int cB = (lane % T::B_CH) ^ b16_swz(kB);
        voffB[j] = kB * ldb * 2 + cB * 16;
    }

    // Global loads of step kt into LDS stage kt % S16, one instruction at a
    // time: stage_desc computes the step's two descriptors, dma_one(j) issues
    // load j (A loads first, then B).  Steps past the end get empty ranges
    // (they only keep the per-step load count uniform).
    struct StageDesc { __amdgpu_buffer_rsrc_t ra, rb; int s; };
    auto stage_desc = [&](int kt) {
        StageDesc d;
        d.s = kt % S16;
        const int k0 = kt * BK16;
        const int krem = K - k0;
        const char* abase = A + ((int64_t)m0 * lda + k0) * 2;
        const int64_t abytes = krem > 0 ? ((int64_t)(rows_a - 1) * lda + krem) * 2 : 0;
        d.ra = make_rsrc(abase, abytes);
        const int rows_b = krem < BK16 ? krem : BK16;
        const char* bbase = B + ((int64_t)k0 * ldb + n0) * 2;
        const int64_t bbytes = rows_b > 0 ? ((int64_t)(rows_b - 1) * ldb + cols_b) * 2 : 0;
        d.rb = make_rsrc(bbase, bbytes);
        return d;
    };
    auto dma_one = [&](const StageDesc& d, int j) {
        if (j < T::A_DMA) {
            dma16(d.ra, lds_addr(smA + d.s * T::A_STAGE + (wave * T::A_DMA + j) * 1024), voffA[j]);
        } else {
            const int jb = j - T::A_DMA;
            dma16(d.rb, lds_addr(smB + d.s * T::B_STAGE + (wave * T::B_DMA + jb) * 1024), voffB[jb]);
        }
    };
    auto issue_stage = [&](int kt) {
        const StageDesc d = stage_desc(kt);
#pragma unroll
        for (int j = 0; j < T::LOADS; ++j) dma_one(d, j);
    };

    // When K is not a multiple of BK16, the last stage's A columns at and past
    // K hold other data (row padding, the next row, or zeros past the range);
    // zero them in LDS so that 0 * (NaN or Inf) can never reach the sum.  B's
    // rows past K are already zero (outside the descriptor's range).
    auto fix_tail = [&]() {
        const int kt = nk - 1;
        const int s = kt % S16;
        const int kin = K - kt * BK16;       // valid k in the last stage, 1..BK16-1
        const int chunk0 = kin >> 3;         // first chunk holding an invalid element
        char* rowp = smA + s * T::A_STAGE;
        const int row = tid;                 // one A row per thread
        if (row < TBM) {
            if (kin & 7) {
                short* p = (short*)(rowp + a16_off(row, chunk0));
                for (int e = kin & 7; e < 8; ++e) p[e] = 0;
            }
            for (int c = chunk0 + ((kin & 7) ? 1 : 0); c < A16_CH; ++c)
                *(u32x4*)(rowp + a16_off(row, c)) = u32x4{0u, 0u, 0u, 0u};
        }
    };

    const int wm = wave >> 1;
    const int wn = wave & 1;
    const int g = lane >> 5;          // lane group: k half of a 16-k chunk pair
    const int li = lane & 31;         // row of A within a 32-row block
    const int ta = (lane >> 2) & 3;   // transpose read: source k row within the group
    const int tq = lane & 3;          // transpose read: source 4-column piece
    const int tg = (lane >> 4) & 1;   // transpose read: the 16-lane group's column half

    f32x16 acc[MI][NJ];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][nj][r] = 0.0f;

    // Operand fragments, one register set per chunk pair of a step: A as
    // MI x 8 consecutive k of a row; B as NJ x (two transpose reads of 4
    // consecutive k of a column).
    u32x4 fa[KP16][MI];
    s16x4 fb[KP16][NJ][2];

    // Fragment read number i (0 .. NREAD - 1) of pair kp of step kt: MI A
    // reads, then 2 NJ B transpose reads (nj = (i - MI) / 2, half (i - MI) % 2).
    auto read_piece = [&](int kt, int kp, u32x4 (&a)[MI], s16x4 (&b)[NJ][2], int i) {
        if (i < MI) {
            const char* sa = smA + (kt % S16) * T::A_STAGE;
            a[i] = *(const u32x4*)(sa + a16_off(wm * (TBM / 2) + i * 32 + li, 2 * kp + g));
        } else {
            const char* sb = smB + (kt % S16) * T::B_STAGE;
            const int nj = (i - MI) >> 1, h = (i - MI) & 1;
            const int k = kp * 16 + 8 * g + 4 * h + ta;
            const int c = wn * (TBN / 16) + nj * 4 + 2 * tg + (tq >> 1);
            b[nj][h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4_t*)(sb + b16_off(k, c, T::B_ROW) + (tq & 1) * 8));
        }
    };
    auto mfma_one = [&](const u32x4 (&a)[MI], const s16x4 (&b)[NJ][2], int mi, int nj) {
        const s16x8 bv = __builtin_shufflevector(b[nj][0], b[nj][1], 0, 1, 2, 3, 4, 5, 6, 7);
        if constexpr (IN == IN_BF16) {
            acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, a[mi]), __builtin_bit_cast(bf16x8, bv), acc[mi][nj], 0, 0, 0);
        } else {
            acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                __builtin_bit_cast(f16x8, a[mi]), __builtin_bit_cast(f16x8, bv), acc[mi][nj], 0, 0, 0);
        }
    };
    auto read_frags = [&](int kt, int kp, u32x4 (&a)[MI], s16x4 (&b)[NJ][2]) {
#pragma unroll
        for (int i = 0; i < T::NREAD; ++i) read_piece(kt, kp, a, b, i);
    };

    // Wait until at most VM of this wave's direct-to-LDS loads are in flight and
    // its LDS accesses are done, then barrier.
    auto sync = [&](auto vm_tag) {
        constexpr int VM = decltype(vm_tag)::value;
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(VM, 0));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    using OneStepLeft = std::integral_constant<int, (S16 - 1) * T::LOADS>;
    using TwoStepsLeft = std::integral_constant<int, (S16 - 2) * T::LOADS>;

    // Schedule (S16 stages, KP16 chunk pairs per step), written out in issue
    // order: with one wave per SIMD nothing else hides a stall, so every
    // load and LDS read sits between two MFMAs (sched_barrier pins the order).
    // Prologue: loads of steps 0 .. S16 - 1.  Step kt: during pair 0's MFMAs
    // read the fragments of pairs 1 .. KP16 - 1 (one register set per pair);
    // then wait until step kt + 1 has landed (later steps may still be in
    // flight) and barrier, which retires every wave's reads of stage kt % S16;
    // then, spread over the MFMAs of pairs 1 .. KP16 - 1, refill that stage
    // with step kt + S16, and during the last pair read pair 0 of step kt + 1.
    if (nk > 0) {
#pragma unroll
        for (int s = 0; s < S16; ++s) issue_stage(s);
        sync(OneStepLeft{});
        if ((K % BK16) && nk == 1) { fix_tail(); sync(OneStepLeft{}); }
        read_frags(0, 0, fa[0], fb[0]);
        for (int kt = 0; kt < nk; ++kt) {
            constexpr int NR = T::NREAD * (KP16 - 1);
#pragma unroll
            for (int i = 0; i < T::NMFMA; ++i) {
                mfma_one(fa[0], fb[0], i / NJ, i % NJ);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int r = (i * NR) / T::NMFMA; r < ((i + 1) * NR) / T::NMFMA; ++r)
                    read_piece(kt, 1 + r / T::NREAD, fa[1 + r / T::NREAD], fb[1 + r / T::NREAD],
                               r % T::NREAD);
                __builtin_amdgcn_sched_barrier(0);
            }
            // Every read of stage kt is now issued: retire them, wait for step
            // kt + 1, barrier.  The stage is then free for step kt + S16.
            const StageDesc d = stage_desc(kt + S16);
            sync(TwoStepsLeft{});
            if ((K % BK16) && kt + 2 == nk) { fix_tail(); sync(TwoStepsLeft{}); }
            const bool more = kt + 1 < nk;
            constexpr int SLOTS = T::NMFMA * (KP16 - 1);
#pragma unroll
            for (int kp = 1; kp < KP16; ++kp) {
#pragma unroll
                for (int i = 0; i < T::NMFMA; ++i) {
                    mfma_one(fa[kp], fb[kp], i / NJ, i % NJ);
                    __builtin_amdgcn_sched_barrier(0);
                    const int slot = (kp - 1) * T::NMFMA + i;
#pragma unroll
                    for (int j = (slot * T::LOADS) / SLOTS; j < ((slot + 1) * T::LOADS) / SLOTS; ++j)
                        dma_one(d, j);
                    __builtin_amdgcn_sched_barrier(0);
                    if (kp == KP16 - 1 && more) {
#pragma unroll
                        for (int r = (i * T::NREAD) / T::NMFMA; r < ((i + 1) * T::NREAD) / T::NMFMA; ++r)
                            read_piece(kt + 1, 0, fa[0], fb[0], r);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    }
    // No direct-to-LDS write may still be in flight when the workgroup ends.
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));

    store_tile<OUT, MI, NJ>(acc, C, M, N, ldc, m0 + wm * (TBM / 2), n0 + wn * (TBN / 2), g, li);
}

// ---------------------------------------------------------------- fp32 kernel

constexpr int ROW_CHUNKS32 = 8;                  // 16-byte chunks per staged row (32 fp32)
constexpr int STAGE_CHUNKS32 = BM * ROW_CHUNKS32;  // one operand's stage: 32 KiB

// LDS slot of chunk c in staged row r.  With phi(r) = (r ^ (r >> 3)) & 7, the 8
// consecutive rows an operand read touches get 8 distinct slots, and so do the
// 8 aligned rows of any 16-row group with equal parity.
__device__ __forceinline__ int lds32_index(int row, int chunk) {
    return row * ROW_CHUNKS32 + (chunk ^ ((row ^ (row >> 3)) & 7));
}

// Zero the fp32 elements of a chunk at and after `valid` (valid <= 0: all).
__device__ __forceinline__ u32x4 mask_tail32(u32x4 v, int valid) {
    u32x4 out;
#pragma unroll
    for (int d = 0; d < 4; ++d) out[d] = (d < valid) ? (uint32_t)v[d] : 0u;
    return out;
}

__global__ __launch_bounds__(NTHREADS) void gemm32_kernel(
    const char* __restrict__ A, const char* __restrict__ B, char* __restrict__ C,
    int M, int N, int K, int lda, int ldb, int ldc, int tiles_m, int tiles_n) {
    // [stage][operand: 0 = A, 1 = B][chunk]: 2 x 2 x 32 KiB.  Both operands are
    // stored K-contiguous: B is transposed on its way through registers.
    __shared__ u32x4 lds[2][2][STAGE_CHUNKS32];

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
    // B staging: thread -> a block of 8 K-rows (kb) by 4 columns (nb).
    const int kb = tid & 3;
    const int nb = tid >> 2;

    int voff_a[8], voff_b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        voff_a[i] = (ar0 + 32 * i) * lda * 4 + ac * 16;
        voff_b[i] = (kb * 8 + i) * ldb * 4 + nb * 16;
    }

    u32x4 ra[8], rb[8];

    auto load_step = [&](int kt, bool tail) {
        const int k0 = kt * BK;
        const char* abase = A + ((int64_t)m0 * lda + k0) * 4;
        const int64_t abytes = ((int64_t)(rows_a - 1) * lda + (K - k0)) * 4;
        const __amdgpu_buffer_rsrc_t rsa = make_rsrc(abase, abytes);
        const int rows_b = (K - k0) < BK ? (K - k0) : BK;
        const char* bbase = B + ((int64_t)k0 * ldb + n0) * 4;
        const int64_t bbytes = ((int64_t)(rows_b - 1) * ldb + cols_b) * 4;
        const __amdgpu_buffer_rsrc_t rsb = make_rsrc(bbase, bbytes);
#pragma unroll
        for (int i = 0; i < 8; ++i) ra[i] = load16(rsa, voff_a[i]);
#pragma unroll
        for (int i = 0; i < 8; ++i) rb[i] = load16(rsb, voff_b[i]);
        if (tail) {
            // Columns of A at or past K hold other data (row padding or the next
            // row); they must be exact zeros, since the matching B rows are.
            const int valid = K - k0 - ac * 4;
#pragma unroll
            for (int i = 0; i < 8; ++i) ra[i] = mask_tail32(ra[i], valid);
        }
    };

    auto store_step = [&](int s) {
#pragma unroll
        for (int i = 0; i < 8; ++i) lds[s][0][lds32_index(ar0 + 32 * i, ac)] = ra[i];
        // 8 K-rows x 4 columns -> 4 columns x two chunks of 4 K values.
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                u32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = rb[4 * h + e][cc];
                lds[s][1][lds32_index(nb * 4 + cc, kb * 2 + h)] = v;
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

    // Operand fragments for one chunk pair (8 k): lane group g reads chunk
    // 2 * kp + g of its 4 A rows and 4 B columns.  Two register sets alternate
    // so that the reads for pair kp + 1 are in flight while kp computes.
    u32x4 fa[2][4], fb[2][4];

    auto read_frags = [&](int s, int kp, u32x4 (&a)[4], u32x4 (&b)[4]) {
        const int ch = 2 * kp + g;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) a[mi] = lds[s][0][lds32_index(wm * 128 + mi * 32 + li, ch)];
#pragma unroll
        for (int nj = 0; nj < 4; ++nj) b[nj] = lds[s][1][lds32_index(wn * 128 + nj * 32 + li, ch)];
    };

    auto mfma_frags = [&](const u32x4 (&a)[4], const u32x4 (&b)[4]) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int nj = 0; nj < 4; ++nj)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                        as_float(a[mi][e]), as_float(b[nj][e]), acc[mi][nj], 0, 0, 0);
    };

    // Schedule of one K step (stage `cur` in LDS, stage cur ^ 1 being filled):
    // global loads for step kt + 1 -> registers; pairs 0, 1, 2: read the next
    // pair's fragments, then compute; registers -> LDS stage cur ^ 1; barrier;
    // read pair 0 of stage cur ^ 1, then compute pair 3 (already in registers),
    // which covers that read's latency.  sched_barrier keeps the compiler from
    // sinking the fragment reads down to their uses.
    if (nk > 0) {
        load_step(0, ragged_k && nk == 1);
        store_step(0);
        __syncthreads();
        read_frags(0, 0, fa[0], fb[0]);
        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            const bool more = kt + 1 < nk;
            if (more) load_step(kt + 1, ragged_k && kt + 2 == nk);
            read_frags(cur, 1, fa[1], fb[1]);
            __builtin_amdgcn_sched_barrier(0);
            mfma_frags(fa[0], fb[0]);
            __builtin_amdgcn_sched_barrier(0);
            read_frags(cur, 2, fa[0], fb[0]);
            __builtin_amdgcn_sched_barrier(0);
            mfma_frags(fa[1], fb[1]);
            __builtin_amdgcn_sched_barrier(0);
            read_frags(cur, 3, fa[1], fb[1]);
            __builtin_amdgcn_sched_barrier(0);
            mfma_frags(fa[0], fb[0]);
            __builtin_amdgcn_sched_barrier(0);
            if (more) store_step(cur ^ 1);
            __syncthreads();
            if (more) read_frags(cur ^ 1, 0, fa[0], fb[0]);
            __builtin_amdgcn_sched_barrier(0);
            mfma_frags(fa[1], fb[1]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    store_tile<OUT_F32>(acc, C, M, N, ldc, m0 + wm * 128, n0 + wn * 128, g, li);
}

// ---------------------------------------------------------------- fp32 via 3 x bf16

// fp32 inputs split into two bf16 parts, x = hi + lo + e with hi = bf16(x),
// lo = bf16(x - hi) (both round to nearest even; x - hi is exact in fp32), so
// |e| <= 2^-16 |x|.  a * b is taken as ah*bh + ah*bl + al*bh: the dropped
// al*bl and the two truncations leave a relative error of at most about
// 3 * 2^-16 per product, before fp32 accumulation.  Three bf16 MFMAs per
// product at 8x the fp32 MFMA rate.
//
// Operands are staged through registers: each thread loads fp32 pieces of A
// (8 consecutive k of one row) and B (an 8 k x 4 column block), splits them,
// and writes hi and lo parts to LDS as K-contiguous bf16 rows (B is transposed
// on the way, by its choice of which values to pack), so both operands are
// read with ds_read_b128.  Double-buffered LDS, BK = 32.

constexpr int X3_ROW = BK * 2;                  // 64-byte bf16 rows: 4 chunks
constexpr int X3_PART = BM * X3_ROW;            // one part of one operand: 16 KiB
constexpr int X3_STAGE = 4 * X3_PART;           // A hi, A lo, B hi, B lo: 64 KiB

__device__ __forceinline__ int x3_off(int row, int chunk) {
    return row * X3_ROW + ((chunk ^ ((row ^ (row >> 2)) & 3)) << 4);
}

// Split 8 fp32 values into packed hi and lo bf16 parts (element i in the low
// half of word i / 2 when i is even).
__device__ __forceinline__ void split8(const float (&x)[8], u32x4& hi, u32x4& lo) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const __bf16 h0 = (__bf16)x[2 * w], h1 = (__bf16)x[2 * w + 1];
        const __bf16 l0 = (__bf16)(x[2 * w] - (float)h0);
        const __bf16 l1 = (__bf16)(x[2 * w + 1] - (float)h1);
        hi[w] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
        lo[w] = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
    }
}

__global__ __launch_bounds__(NTHREADS) void gemm32x3_kernel(
    const char* __restrict__ A, const char* __restrict__ B, char* __restrict__ C,
    int M, int N, int K, int lda, int ldb, int ldc, int tiles_m, int tiles_n) {
    __shared__ __attribute__((aligned(1024))) char smem[2 * X3_STAGE];

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

    // A staging: thread -> 8 consecutive k (two 16-byte fp32 pieces) of rows
    // ar0 + 64 i, i = 0..3, k chunk ac.
    const int ac = tid & 3;
    const int ar0 = tid >> 2;
    // B staging: thread -> an 8 k x 4 column block (k rows 8 kb .., columns 4 nb ..).
    const int kb = tid & 3;
    const int nb = tid >> 2;

    int voff_a[4], voff_b[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) voff_a[i] = (ar0 + 64 * i) * lda * 4 + ac * 32;
#pragma unroll
    for (int i = 0; i < 8; ++i) voff_b[i] = (kb * 8 + i) * ldb * 4 + nb * 16;

    u32x4 ra[8], rb[8];

    auto load_step = [&](int kt, bool tail) {
        const int k0 = kt * BK;
        const char* abase = A + ((int64_t)m0 * lda + k0) * 4;
        const int64_t abytes = ((int64_t)(rows_a - 1) * lda + (K - k0)) * 4;
        const __amdgpu_buffer_rsrc_t rsa = make_rsrc(abase, abytes);
        const int rows_b = (K - k0) < BK ? (K - k0) : BK;
        const char* bbase = B + ((int64_t)k0 * ldb + n0) * 4;
        const int64_t bbytes = ((int64_t)(rows_b - 1) * ldb + cols_b) * 4;
        const __amdgpu_buffer_rsrc_t rsb = make_rsrc(bbase, bbytes);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ra[2 * i] = load16(rsa, voff_a[i]);
            ra[2 * i + 1] = load16(rsa, voff_a[i] + 16);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) rb[i] = load16(rsb, voff_b[i]);
        if (tail) {
            // Columns of A at or past K hold other data (row padding or the next
            // row); they must be exact zeros, since the matching B rows are.
            const int valid = K - k0 - ac * 8;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ra[2 * i] = mask_tail32(ra[2 * i], valid);
                ra[2 * i + 1] = mask_tail32(ra[2 * i + 1], valid - 4);
            }
        }
    };

    auto store_step = [&](int s) {
        char* st = smem + s * X3_STAGE;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[e] = as_float(ra[2 * i][e]);
                x[4 + e] = as_float(ra[2 * i + 1][e]);
            }
            u32x4 hi, lo;
            split8(x, hi, lo);
            const int off = x3_off(ar0 + 64 * i, ac);
            *(u32x4*)(st + off) = hi;
            *(u32x4*)(st + X3_PART + off) = lo;
        }
        // B: column cc of the block, 8 consecutive k -> one chunk per part.
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = as_float(rb[e][cc]);
            u32x4 hi, lo;
            split8(x, hi, lo);
            const int off = x3_off(nb * 4 + cc, kb);
            *(u32x4*)(st + 2 * X3_PART + off) = hi;
            *(u32x4*)(st + 3 * X3_PART + off) = lo;
        }
    };

    const int wm = wave >> 1;
    const int wn = wave & 1;
    const int g = lane >> 5;
    const int li = lane & 31;

    f32x16 acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int nj = 0; nj < 4; ++nj)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][nj][r] = 0.0f;

    // Fragments of one 16-k chunk pair: [part][block], part 0 = hi, 1 = lo.
    u32x4 fa[2][2][4], fb[2][2][4];

    auto read_frags = [&](int s, int kp, u32x4 (&a)[2][4], u32x4 (&b)[2][4]) {
        const char* st = smem + s * X3_STAGE;
        const int ch = 2 * kp + g;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
                a[p][mi] = *(const u32x4*)(st + p * X3_PART + x3_off(wm * 128 + mi * 32 + li, ch));
#pragma unroll
            for (int nj = 0; nj < 4; ++nj)
                b[p][nj] = *(const u32x4*)(st + (2 + p) * X3_PART + x3_off(wn * 128 + nj * 32 + li, ch));
        }
    };

    auto mfma_frags = [&](const u32x4 (&a)[2][4], const u32x4 (&b)[2][4]) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
            for (int nj = 0; nj < 4; ++nj) {
                // small terms first, then the leading one
                acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, a[1][mi]), __builtin_bit_cast(bf16x8, b[0][nj]), acc[mi][nj], 0, 0, 0);
                acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, a[0][mi]), __builtin_bit_cast(bf16x8, b[1][nj]), acc[mi][nj], 0, 0, 0);
                acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, a[0][mi]), __builtin_bit_cast(bf16x8, b[0][nj]), acc[mi][nj], 0, 0, 0);
            }
        }
    };

    // Per step: global loads of step kt + 1 -> registers; read pair 1 while
    // pair 0 computes; split and write step kt + 1 to the other stage;
    // barrier; read pair 0 of step kt + 1 while pair 1 computes.
    if (nk > 0) {
        load_step(0, ragged_k && nk == 1);
        store_step(0);
        __syncthreads();
        read_frags(0, 0, fa[0], fb[0]);
        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            const bool more = kt + 1 < nk;
            if (more) load_step(kt + 1, ragged_k && kt + 2 == nk);
            read_frags(cur, 1, fa[1], fb[1]);
            __builtin_amdgcn_sched_barrier(0);
            mfma_frags(fa[0], fb[0]);
            __builtin_amdgcn_sched_barrier(0);
            if (more) store_step(cur ^ 1);
            __syncthreads();
            if (more) read_frags(cur ^ 1, 0, fa[0], fb[0]);
            __builtin_amdgcn_sched_barrier(0);
            mfma_frags(fa[1], fb[1]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    store_tile<OUT_F32>(acc, C, M, N, ldc, m0 + wm * 128, n0 + wn * 128, g, li);
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
             int ldc, int in, int es_out) {
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
    if ((int64_t)BM * lda * es >= DESC_LIMIT || (int64_t)BK * ldb * es >= DESC_LIMIT)
        return DGEMM_ERR_TOO_LARGE;
    return DGEMM_OK;
}

// Macro-tile choice for the 16-bit kernel: the candidate minimising the
// estimated time ceil(tiles / CUs) x tile_area / efficiency, where the
// efficiencies (256 x 256: 1, 192 x 256: 0.95, 128 x 128: 0.6) are rough
// measured ratios of per-tile throughput.  Large grids keep 256 x 256; grids
// that would leave CUs idle (4000 x 3000: 192 tiles of 256^2 against 252 of
// 192 x 256) or that have few tiles (512^2) move to smaller tiles.  fp32
// kernels use 256 x 256 only.  Fixed CU count: the choice does not depend on
// the device, so the host query below reports exactly what a launch uses.
constexpr int NUM_CU = 256;

struct TileChoice { int bm, bn; };

TileChoice pick_tile(int in, int M, int N) {
    if (in == IN_F32 || in == IN_F32X3) return {BM, BN};
    const struct { int bm, bn; double eff; } cand[] = {{256, 256, 1.0}, {192, 256, 0.95}, {128, 128, 0.6}};
    TileChoice best{256, 256};
    double best_cost = -1.0;
    for (const auto& c : cand) {
        const int64_t tiles = (((int64_t)M + c.bm - 1) / c.bm) * (((int64_t)N + c.bn - 1) / c.bn);
        const int64_t waves = (tiles + NUM_CU - 1) / NUM_CU;
        const double cost = (double)waves * c.bm * c.bn / c.eff;
        if (best_cost < 0 || cost < best_cost) { best_cost = cost; best = {c.bm, c.bn}; }
    }
    return best;
}

template <int IN, int OUT, int TBM, int TBN>
const void* kernel_for() {
    if constexpr (IN == IN_F32)
        return (const void*)gemm32_kernel;
    else if constexpr (IN == IN_F32X3)
        return (const void*)gemm32x3_kernel;
    else
        return (const void*)gemm16_kernel<IN, OUT, TBM, TBN>;
}

template <int IN, int OUT>
int launch(int M, int N, int K, const void* A, int lda, const void* B, int ldb, void* C, int ldc,
           void* stream) {
    const TileChoice t = pick_tile(IN, M, N);
    int tiles_m = (M + t.bm - 1) / t.bm;
    int tiles_n = (N + t.bn - 1) / t.bn;
    const int64_t ntiles = (int64_t)tiles_m * tiles_n;
    if (ntiles > INT32_MAX) return DGEMM_ERR_TOO_LARGE;
    const char* a = (const char*)A;
    const char* b = (const char*)B;
    char* c = (char*)C;
    void* args[] = {&a, &b, &c, &M, &N, &K, &lda, &ldb, &ldc, &tiles_m, &tiles_n};
    const void* fn;
    if (t.bm == 256)
        fn = kernel_for<IN, OUT, 256, 256>();
    else if (t.bm == 192)
        fn = kernel_for<IN, OUT, 192, 256>();
    else
        fn = kernel_for<IN, OUT, 128, 128>();
    hipError_t e = hipLaunchKernel(fn, dim3((unsigned)ntiles), dim3(NTHREADS), args, 0,
                                   (hipStream_t)stream);
    return e == hipSuccess ? DGEMM_OK : DGEMM_ERR_LAUNCH;
}

template <int IN>
int gemm_entry(int M, int N, int K, const void* A, int lda, const void* B, int ldb, void* C,
               int ldc, int out, void* stream) {
    if (out != DGEMM_OUT_F32 && out != DGEMM_OUT_SAME) return DGEMM_ERR_INVALID_VALUE;
    const int es_out = out == DGEMM_OUT_F32 ? 4 : in_esize(IN);
    int st = validate(M, N, K, A, lda, B, ldb, C, ldc, IN, es_out);
    if (st != DGEMM_OK) return st;
    if (M == 0 || N == 0) return DGEMM_OK;
    st = check_device();
    if (st != DGEMM_OK) return st;
    if (out == DGEMM_OUT_F32) return launch<IN, OUT_F32>(M, N, K, A, lda, B, ldb, C, ldc, stream);
    if constexpr (IN == IN_F32 || IN == IN_F32X3)
        return DGEMM_ERR_INVALID_VALUE;  // fp32 inputs always give fp32 C
    else if constexpr (IN == IN_BF16)
        return launch<IN_BF16, OUT_BF16>(M, N, K, A, lda, B, ldb, C, ldc, stream);
    else
        return launch<IN_F16, OUT_F16>(M, N, K, A, lda, B, ldb, C, ldc, stream);
}

}  // namespace

extern "C" {

int gemm_f32(int M, int N, int K, const float* A, int lda, const float* B, int ldb, float* C,
             int ldc, void* stream) {
    return gemm_entry<IN_F32>(M, N, K, A, lda, B, ldb, C, ldc, DGEMM_OUT_F32, stream);
}

int gemm_f32_3xbf16(int M, int N, int K, const float* A, int lda, const float* B, int ldb,
                    float* C, int ldc, void* stream) {
    return gemm_entry<IN_F32X3>(M, N, K, A, lda, B, ldb, C, ldc, DGEMM_OUT_F32, stream);
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
    if (M < 0 || N < 0 || (in != IN_F32 && in != IN_BF16 && in != IN_F16 && in != IN_F32X3))
        return DGEMM_ERR_INVALID_VALUE;
    const TileChoice t = pick_tile(in, M, N);
    const int64_t tm_count = ((int64_t)M + t.bm - 1) / t.bm;
    const int64_t tn_count = ((int64_t)N + t.bn - 1) / t.bn;
    if (tm_count * tn_count > INT32_MAX) return DGEMM_ERR_TOO_LARGE;
    const int nwg = (int)(tm_count * tn_count);
    if (tile_rows) *tile_rows = t.bm;
    if (tile_cols) *tile_cols = t.bn;
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
