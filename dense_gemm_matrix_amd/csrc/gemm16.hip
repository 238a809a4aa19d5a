// gemm16.hip -- the bf16 / fp16 GEMM kernel for gfx950 (MI355X).
//
// Both operands go global -> LDS with direct-to-LDS buffer loads (no VGPR
// staging, no LDS write instructions) into a ring of S stages of BK16 = 64-deep
// slabs, each issued S - 1 steps before its use.  S = 2 for the 256-wide tiles
// (of the settings that fit 160 KiB, measured fastest; 4 x 32 and 5 x 32 deep
// were slower).  The 128 x 128 tile has both S = 2 (64 KiB: two workgroups per
// CU, each hiding the other's load latency) and S = 4 (128 KiB: one workgroup
// per CU, loads issued three steps ahead); the planner takes S = 4 when the
// grid has no more workgroups than CUs.  A is stored K-contiguous and read with ds_read_b128.  B is stored as it
// lies in memory (row-major, N-contiguous) and read with ds_read_b64_tr_b16:
// within each 16-lane group that instruction performs a 4 x 4 transpose of
// 4-element row pieces, which hands every lane the four consecutive k of one
// column that the matrix instruction's B operand needs.
// v_mfma_f32_32x32x16_{bf16,f16}, fp32 accumulators.
//
// Per workgroup as launched: 256 threads = 4 waves of 64 lanes in a 2 x 2
// layout, one wave per SIMD, each wave owning a (TBM/2) x (TBN/2) sub-tile held
// as blocks of 32 x 32 accumulators (256 fp32 per lane at 256 x 256,
// register-resident for the whole K loop).  The template also builds a 2 x 4
// layout of 8 waves (two per SIMD), which measured slower at 4096^3.  LDS rows are split into 16-byte chunks whose positions are
// XORed with a function of the row, so every 16-byte access stays aligned (the
// principle of the sgemm tf32 page's section 3 swizzles and the hgemm page's
// section 2) while the access patterns used here hit distinct LDS banks.  The
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

#include "kern_common.h"

namespace dgemm {
namespace {

constexpr int BK16 = 64;                       // K per stage
constexpr int KP16 = BK16 / 16;                // 16-k chunk pairs per stage
constexpr int A16_CH = BK16 / 8;               // 16-byte chunks per A row
constexpr int A16_ROW = BK16 * 2;              // bytes per staged A row
constexpr int A16_RPB = 1024 / A16_ROW;        // A rows per 1 KiB load block

// Macro-tile TBM x TBN, 2 x WN waves (WN = 2: 4 waves, one per SIMD; WN = 4:
// 8 waves, two per SIMD), each wave (TBM/2) x (TBN/WN) = MI x NJ blocks of
// 32 x 32 accumulators, and an LDS ring of S stages.
template <int TBM, int TBN, int WN = 2, int S_ = 2>
struct Tile16 {
    static constexpr int S = S_;                         // LDS stages
    static constexpr int NW = 2 * WN;                    // waves
    static constexpr int NT = 64 * NW;                   // threads
    static constexpr int MI = TBM / 64;
    static constexpr int NJ = TBN / (32 * WN);
    static constexpr int A_STAGE = TBM * A16_ROW;        // bytes per A stage
    static constexpr int B_ROW = TBN * 2;                // bytes per staged B row
    static constexpr int B_CH = TBN / 8;                 // 16-byte chunks per B row
    static constexpr int B_STAGE = BK16 * B_ROW;         // bytes per B stage
    static constexpr int B_RPB = 1024 / B_ROW;           // B rows per 1 KiB load block
    static constexpr int A_DMA = A_STAGE / 1024 / NW;    // direct-to-LDS loads per wave per stage
    static constexpr int B_DMA = B_STAGE / 1024 / NW;
    static constexpr int LOADS = A_DMA + B_DMA;
    static constexpr int NREAD = MI + 2 * NJ;            // fragment reads per chunk pair
    static constexpr int NMFMA = MI * NJ;                // MFMAs per chunk pair
    static_assert(TBM % 64 == 0 && TBN % (32 * WN) == 0 && TBM <= NT, "tile shape");
    static_assert(A_STAGE % (1024 * NW) == 0 && B_STAGE % (1024 * NW) == 0,
                  "whole load blocks per wave");
    static_assert(S * (A_STAGE + B_STAGE) <= 160 * 1024, "LDS budget");
    static_assert(S >= 2 && (S - 1) * LOADS <= 63, "stages, vmcnt range");
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

template <int IN, int OUT, int TBM, int TBN, bool EPI, int WN, int S>
__global__ __launch_bounds__((Tile16<TBM, TBN, WN, S>::NT)) void gemm16_kernel(
    const char* __restrict__ A, const char* __restrict__ B, char* __restrict__ C,
    int M, int N, int K, int lda, int ldb, int ldc, int tiles_m, int tiles_n,
    int kchunk, int64_t c_zstride, EpiArgs epi) {
    using T = Tile16<TBM, TBN, WN, S>;
    // Split-K: workgroup row z of the grid covers k in [z kchunk, (z+1) kchunk)
    // and writes its partial sums at C + z c_zstride (z = 0, kchunk = K when unsplit).
    {
        const int z = (int)blockIdx.y;
        const int kbeg = z * kchunk;
        A += (int64_t)kbeg * 2;
        B += (int64_t)kbeg * ldb * 2;
        C += z * c_zstride;
        K = (K - kbeg) < kchunk ? (K - kbeg) : kchunk;
    }
    constexpr int MI = T::MI, NJ = T::NJ;
    __shared__ __attribute__((aligned(1024))) char smem[T::S * (T::A_STAGE + T::B_STAGE)];
    char* const smA = smem;
    char* const smB = smem + T::S * T::A_STAGE;

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

    // Global loads of step kt into LDS stage kt % S, one instruction at a
    // time: stage_desc computes the step's two descriptors, dma_one(j) issues
    // load j (A loads first, then B).  Steps past the end get empty ranges
    // (they only keep the per-step load count uniform).
    struct StageDesc { __amdgpu_buffer_rsrc_t ra, rb; int s; };
    auto stage_desc = [&](int kt) {
        StageDesc d;
        d.s = kt % T::S;
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
        const int s = kt % T::S;
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

    const int wm = wave / WN;
    const int wn = wave % WN;
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
            const char* sa = smA + (kt % T::S) * T::A_STAGE;
            a[i] = *(const u32x4*)(sa + a16_off(wm * (TBM / 2) + i * 32 + li, 2 * kp + g));
        } else {
            const char* sb = smB + (kt % T::S) * T::B_STAGE;
            const int nj = (i - MI) >> 1, h = (i - MI) & 1;
            const int k = kp * 16 + 8 * g + 4 * h + ta;
            const int c = wn * (TBN / WN / 8) + nj * 4 + 2 * tg + (tq >> 1);
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
    // Block column of MFMA i of a chunk pair: rows in turn, odd rows right to
    // left, so consecutive MFMAs always share one operand register set (the
    // row-major order changes both at each new row).  Fewer operand bits change
    // per instruction; at the board's power limit that measured ~0.5 % faster.
    // Each accumulator still sees its k in the same order: the same results.
    auto snake = [](int i) { return ((i / NJ) & 1) ? NJ - 1 - i % NJ : i % NJ; };
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
    using OneStepLeft = std::integral_constant<int, (T::S - 1) * T::LOADS>;
    using TwoStepsLeft = std::integral_constant<int, (T::S - 2) * T::LOADS>;

    // Schedule (S stages, KP16 chunk pairs per step), written out in issue
    // order: with one wave per SIMD nothing else hides a stall, so every
    // load and LDS read sits between two MFMAs (sched_barrier pins the order).
    // Prologue: loads of steps 0 .. S - 1.  Step kt: spread over the MFMAs
    // of pairs 0 and 1, read the fragments of pairs 1 .. KP16 - 1 (one
    // register set per pair; each pair's reads are issued before its MFMAs
    // start); then wait until step kt + 1 has landed (later steps may still be
    // in flight) and barrier, which retires every wave's reads of stage
    // kt % S; then, spread over the MFMAs of pairs 2 .. KP16 - 1, refill that
    // stage with step kt + S and read pair 0 of step kt + 1 (its stage landed
    // before the barrier, and pair 0's registers are free).  Spreading those
    // reads over both pairs rather than the last one measured 1-4 % faster on
    // the tiles that are not power-limited.  (A barrier after pair 0, with the
    // refill over three pairs, measured about 1 % slower.)
    // The last step reads that pair too (from the stage the empty loads past
    // K have zero-filled, inside the LDS array; the registers are never
    // used): an unconditional read saves a branch per matrix instruction.
    if (nk > 0) {
#pragma unroll
        for (int s = 0; s < T::S; ++s) issue_stage(s);
        sync(OneStepLeft{});
        if ((K % BK16) && nk == 1) { fix_tail(); sync(OneStepLeft{}); }
        read_frags(0, 0, fa[0], fb[0]);
        for (int kt = 0; kt < nk; ++kt) {
            constexpr int NR = T::NREAD * (KP16 - 1);
#pragma unroll
            for (int i = 0; i < 2 * T::NMFMA; ++i) {
                if (i < T::NMFMA) mfma_one(fa[0], fb[0], i / NJ, snake(i));
                else mfma_one(fa[1], fb[1], (i - T::NMFMA) / NJ, snake(i - T::NMFMA));
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int r = (i * NR) / (2 * T::NMFMA); r < ((i + 1) * NR) / (2 * T::NMFMA); ++r)
                    read_piece(kt, 1 + r / T::NREAD, fa[1 + r / T::NREAD], fb[1 + r / T::NREAD],
                               r % T::NREAD);
                __builtin_amdgcn_sched_barrier(0);
            }
            // Every read of stage kt is now issued: retire them, wait for step
            // kt + 1, barrier.  The stage is then free for step kt + S.
            const StageDesc d = stage_desc(kt + T::S);
            sync(TwoStepsLeft{});
            if ((K % BK16) && kt + 2 == nk) { fix_tail(); sync(TwoStepsLeft{}); }
            constexpr int SLOTS = T::NMFMA * (KP16 - 2);
#pragma unroll
            for (int kp = 2; kp < KP16; ++kp) {
#pragma unroll
                for (int i = 0; i < T::NMFMA; ++i) {
                    mfma_one(fa[kp], fb[kp], i / NJ, snake(i));
                    __builtin_amdgcn_sched_barrier(0);
                    const int slot = (kp - 2) * T::NMFMA + i;
#pragma unroll
                    for (int j = (slot * T::LOADS) / SLOTS; j < ((slot + 1) * T::LOADS) / SLOTS; ++j)
                        dma_one(d, j);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int r = (slot * T::NREAD) / SLOTS; r < ((slot + 1) * T::NREAD) / SLOTS; ++r)
                        read_piece(kt + 1, 0, fa[0], fb[0], r);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    }
    // No direct-to-LDS write may still be in flight when the workgroup ends.
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));

    store_tile<OUT, MI, NJ, EPI>(acc, C, M, N, ldc, m0 + wm * (TBM / 2), n0 + wn * (TBN / WN), g, li,
                                 epi, m0 + TBM <= M && n0 + TBN <= N);
}

template <int IN, int OUT, int TBM, int TBN, bool EPI, int WN = 2, int S = 2>
hipError_t go(const GemmLaunch& L) {
    const char* a = L.A;
    const char* b = L.B;
    char* c = L.C;
    int M = L.M, N = L.N, K = L.K, lda = L.lda, ldb = L.ldb, ldc = L.ldc;
    int tiles_m = L.tiles_m, tiles_n = L.tiles_n, kchunk = L.kchunk;
    int64_t zs = L.c_zstride;
    EpiArgs e = L.e;
    void* args[] = {&a, &b, &c, &M, &N, &K, &lda, &ldb, &ldc, &tiles_m, &tiles_n, &kchunk, &zs, &e};
    return hipLaunchKernel((const void*)gemm16_kernel<IN, OUT, TBM, TBN, EPI, WN, S>,
                           dim3((unsigned)(tiles_m * tiles_n), (unsigned)L.splits),
                           dim3(Tile16<TBM, TBN, WN, S>::NT),
                           args, 0, L.stream);
}

template <int IN, int OUT, bool EPI>
hipError_t by_tile(const GemmLaunch& L) {
    if (L.tbm == 256 && L.tbn == 256) return go<IN, OUT, 256, 256, EPI>(L);
    if (L.tbm == 192 && L.tbn == 256) return go<IN, OUT, 192, 256, EPI>(L);
    if (L.tbm == 128 && L.tbn == 128)
        return L.stages == 4 ? go<IN, OUT, 128, 128, EPI, 2, 4>(L) : go<IN, OUT, 128, 128, EPI, 2, 2>(L);
    return hipErrorInvalidValue;
}

template <int IN, int OUT>
hipError_t by_epi(const GemmLaunch& L) {
    return L.epi ? by_tile<IN, OUT, true>(L) : by_tile<IN, OUT, false>(L);
}

}  // namespace

hipError_t launch_gemm16(const GemmLaunch& L) {
    if (L.in == IN_BF16) {
        if (L.out == OUT_F32) return by_epi<IN_BF16, OUT_F32>(L);
        if (L.out == OUT_BF16) return by_epi<IN_BF16, OUT_BF16>(L);
    } else if (L.in == IN_F16) {
        if (L.out == OUT_F32) return by_epi<IN_F16, OUT_F32>(L);
        if (L.out == OUT_F16) return by_epi<IN_F16, OUT_F16>(L);
    }
    return hipErrorInvalidValue;
}

}  // namespace dgemm
