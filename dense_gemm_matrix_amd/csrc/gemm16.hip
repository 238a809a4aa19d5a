// gemm16.hip -- the bf16 / fp16 GEMM kernel for gfx950 (MI355X).
//
// Both operands go global -> LDS with direct-to-LDS buffer loads (no VGPR
// staging, no LDS write instructions).  A is staged in slabs of BKA = 64 k, so
// that every A row piece a load fetches is one 128-byte cache line (64-byte
// pieces measured 1.5x the L1 -> L2 read requests and twice the L1's
// pending-request stalls), stored K-contiguous and read with ds_read_b128.  B
// is stored as it lies in memory (row-major, N-contiguous) and read with
// ds_read_b64_tr_b16: within each 16-lane group that instruction performs a
// 4 x 4 transpose of 4-element row pieces, which hands every lane the four
// consecutive k of one column that the matrix instruction's B operand needs.
// v_mfma_f32_32x32x16_{bf16,f16}, fp32 accumulators.
//
// Two schedules of the K loop, chosen per macro-tile by what measured faster:
//   SLAB2 (256 x 256, 128 x 128): steps of 64 k; a ring of S stages of A and
//     B (S = 2, or 4 for the 128 x 128 tile alone on its CU) with one barrier
//     per step, placed after half of the step's matrix instructions; the next
//     stage's loads go out in the second half.  The 256 x 256 tile runs at the
//     board's power limit, where this schedule measured 4-5 % faster than RING.
//   RING (192 x 256): steps of 32 k; SA = 3 A slabs and SB = 2 SA - 2 = 4 B
//     stages of 32 k-rows (136 KiB), a barrier at the top of each step, and
//     each step's loads (half an A slab and a B stage, SB - 1 steps ahead)
//     spread evenly over all of the step's matrix instructions.  That tile is
//     not power-limited, and there this schedule measured 3-4 % faster.
//
// Per workgroup as launched: 256 threads = 4 waves of 64 lanes in a 2 x 2
// layout, one wave per SIMD, each wave owning a (TBM/2) x (TBN/2) sub-tile held
// as blocks of 32 x 32 accumulators (256 fp32 per lane at 256 x 256,
// register-resident for the whole K loop).  LDS rows are split into 16-byte
// chunks whose positions are XORed with a function of the row, so every
// 16-byte access stays aligned (the principle of the sgemm tf32 page's
// section 3 swizzles and the hgemm page's section 2) while the access patterns
// used here hit distinct LDS banks.  The bijective workgroup -> tile map keeps
// each XCD's workgroups on a compact block of tiles (the sgemm tf32 page's
// section 4 Grid Swizzling, adapted to 8 XCDs with private L2s).  Buffer loads
// use per-stage resource descriptors: rows past M (A) and past K (B) fall
// outside the range and read as zero, A's K tail is forced to exact zeros, and
// the epilogue stores only inside M x N; no host padding (the nine-levels
// tutorial's sections 2.9 and 6.1 offer padding or predication; predication
// is chosen).
//
// Matrix instructions' internal k order is not observable through the ABI: a
// lane group's operand carries the same k indices for A and for B, so any
// permutation of k inside an instruction cancels.

#include <type_traits>

#include "kern_common.h"

namespace dgemm {
namespace {

constexpr int BKA = 64;                        // K per A slab
constexpr int A16_CH = BKA / 8;                // 16-byte chunks per A row
constexpr int A16_ROW = BKA * 2;               // bytes per staged A row
constexpr int A16_RPB = 1024 / A16_ROW;        // A rows per 1 KiB load block

enum Sched16 { SLAB2 = 0, RING = 1 };

// Macro-tile TBM x TBN, 4 waves in a 2 x 2 layout, each wave (TBM/2) x (TBN/2)
// = MI x NJ blocks of 32 x 32 accumulators.  SLAB2: SA stages of 64 k of both
// operands.  RING: SA A slabs of 64 k and SB = 2 SA - 2 B stages of 32 k.
template <int TBM, int TBN, int SCHED, int SA_>
struct Tile16 {
    static constexpr bool R = SCHED == RING;
    static constexpr int SA = SA_;                       // A slabs
    static constexpr int SB = R ? 2 * SA - 2 : SA;       // B stages
    static constexpr int STEPK = R ? 32 : 64;            // K per loop step (= per B stage)
    static constexpr int KP = STEPK / 16;                // 16-k chunk pairs per step
    static constexpr int NW = 4;                         // waves
    static constexpr int MI = TBM / 64;
    static constexpr int NJ = TBN / 64;
    static constexpr int A_STAGE = TBM * A16_ROW;        // bytes per A slab
    static constexpr int B_ROW = TBN * 2;                // bytes per staged B row
    static constexpr int B_CH = TBN / 8;                 // 16-byte chunks per B row
    static constexpr int B_STAGE = STEPK * B_ROW;        // bytes per B stage
    static constexpr int B_RPB = 1024 / B_ROW;           // B rows per 1 KiB load block
    static constexpr int AH = R ? 2 : 1;                 // steps that load one A slab
    static constexpr int A_DMA = A_STAGE / 1024 / NW / AH;  // A loads per wave per step
    static constexpr int B_DMA = B_STAGE / 1024 / NW;       // B loads per wave per step
    static constexpr int LOADS = A_DMA + B_DMA;
    static constexpr int NREAD = MI + 2 * NJ;            // fragment reads per chunk pair
    static constexpr int NMFMA = MI * NJ;                // MFMAs per chunk pair
    static constexpr int LDS = SA * A_STAGE + SB * B_STAGE;
    static_assert(TBM % 64 == 0 && TBN % 64 == 0 && TBM <= 64 * NW, "tile shape");
    static_assert(A_STAGE % (1024 * NW * AH) == 0 && B_STAGE % (1024 * NW) == 0,
                  "whole load blocks per wave");
    static_assert(LDS <= 160 * 1024, "LDS budget");
    static_assert(R ? (SA >= 3 && (2 * SA - 4) * LOADS <= 63) : (SA >= 2 && (SA - 1) * LOADS <= 63),
                  "stages, vmcnt range");
    static_assert(NREAD <= 15, "lgkmcnt range");
};

// Byte offset of chunk c (0..7) of A row r in a slab.  ds_read_b128 serves
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

// The K loop of one macro-tile: acc := A[m0 .. m0 + TBM) x B[.., n0 .. n0 + TBN)
// over k in [0, K), with A and B already offset to the first k and rows_a /
// cols_b the tile's rows of A and columns of B inside the matrices (ZERO =
// false: acc += that product, the matrix instructions accumulating onto acc's
// values).  smem is the workgroup's LDS ring (Tile16::LDS bytes).  Every wave
// of the workgroup calls it together; on return no load or LDS access of this
// wave is in flight, but other waves may still be reading the ring.
template <int IN, int TBM, int TBN, int SCHED, int S, bool ZERO = true, bool PER_CALL = false>
__device__ __forceinline__ void mainloop16(const char* __restrict__ A, const char* __restrict__ B,
                                           int K, int lda, int ldb, int m0, int n0, int rows_a,
                                           int cols_b, char* smem,
                                           f32x16 (&acc)[TBM / 64][TBN / 64]) {
    using T = Tile16<TBM, TBN, SCHED, S>;
    constexpr bool RINGS = T::R;
    constexpr int MI = T::MI, NJ = T::NJ;
    char* const smA = smem;
    char* const smB = smem + T::SA * T::A_STAGE;
    int tid = (int)threadIdx.x;
    // PER_CALL (a caller that runs several K loops): make the lane's offsets
    // opaque per call, so the compiler derives them inside each call rather
    // than keeping them in registers across the caller's loop.
    if constexpr (PER_CALL) asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in an SGPR
    const int nk = (K + T::STEPK - 1) / T::STEPK;   // loop steps

    // Each direct-to-LDS instruction fills a 1 KiB block lane-linearly (lane l
    // -> bytes 16 l .. 16 l + 15), so the swizzle is applied on the global side:
    // lane l fetches the chunk that belongs in its slot.  An A slab's blocks are
    // A16_RPB rows of A16_CH chunks; wave w fills blocks AH w A_DMA ..
    // AH (w + 1) A_DMA - 1 (under RING half of them, h = 0, 1, in each of the
    // two steps that load the slab).  A B stage's blocks are B_RPB k-rows of
    // B_CH chunks; wave w fills blocks w B_DMA .. (w + 1) B_DMA - 1.
    int voffA[T::AH][T::A_DMA], voffB[T::B_DMA];
#pragma unroll
    for (int h = 0; h < T::AH; ++h)
#pragma unroll
        for (int j = 0; j < T::A_DMA; ++j) {
            const int rowA = ((T::AH * wave + h) * T::A_DMA + j) * A16_RPB + lane / A16_CH;
            const int cA = (lane % A16_CH) ^ a16_phi(rowA);
            voffA[h][j] = rowA * lda * 2 + cA * 16;
        }
#pragma unroll
    for (int j = 0; j < T::B_DMA; ++j) {
        const int kB = (wave * T::B_DMA + j) * T::B_RPB + lane / T::B_CH;
        const int cB = (lane % T::B_CH) ^ b16_swz(kB);
        voffB[j] = kB * ldb * 2 + cB * 16;
    }

    // Descriptors and ring slots of A slab v and B stage j.  Slabs and stages
    // past the end get empty ranges (their loads keep the per-step load count
    // uniform and fill zeros).  dma_one(j) issues load j of a step (A loads
    // first, then B); h (which half of the A slab, RING) is a compile-time
    // constant at every call, so voffA is indexed statically.
    struct LoadDesc { __amdgpu_buffer_rsrc_t ra, rb; int sa, sb; };
    auto load_desc = [&](int v, int j) {
        LoadDesc d;
        d.sa = v % T::SA;
        d.sb = (j + T::SB) % T::SB;
        const int ka = v * BKA;
        const int krem_a = K - ka;
        const char* abase = A + ((int64_t)m0 * lda + ka) * 2;
        const int64_t abytes =
            krem_a > 0 ? ((int64_t)(rows_a - 1) * lda + (krem_a < BKA ? krem_a : BKA)) * 2 : 0;
        d.ra = make_rsrc(abase, abytes);
        const int kb = j * T::STEPK;
        const int rows_b = (K - kb) < T::STEPK ? (K - kb) : T::STEPK;
        const char* bbase = B + ((int64_t)kb * ldb + n0) * 2;
        const int64_t bbytes = rows_b > 0 ? ((int64_t)(rows_b - 1) * ldb + cols_b) * 2 : 0;
        d.rb = make_rsrc(bbase, bbytes);
        return d;
    };
    auto dma_one = [&](const LoadDesc& d, int h, int j) {
        if (j < T::A_DMA) {
            const int blk = (T::AH * wave + h) * T::A_DMA + j;
            dma16(d.ra, lds_addr(smA + d.sa * T::A_STAGE + blk * 1024), voffA[h][j]);
        } else {
            const int jb = j - T::A_DMA;
            dma16(d.rb, lds_addr(smB + d.sb * T::B_STAGE + (wave * T::B_DMA + jb) * 1024), voffB[jb]);
        }
    };

    // When K is not a multiple of BKA, the last A slab's columns at and past K
    // hold other data (row padding, the next row, or zeros past the range);
    // zero them in LDS so that 0 * (NaN or Inf) can never reach the sum.  B's
    // rows past K are already zero (outside the descriptor's range).
    const int last_slab = (K - 1) / BKA;
    auto fix_tail = [&]() {
        const int kin = K - last_slab * BKA;  // valid k in the last slab, 1..BKA-1
        const int chunk0 = kin >> 3;          // first chunk holding an invalid element
        char* rowp = smA + (last_slab % T::SA) * T::A_STAGE;
        const int row = tid;                  // one A row per thread
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

    if constexpr (ZERO) {
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int nj = 0; nj < NJ; ++nj)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[mi][nj][r] = 0.0f;
    }

    // Operand fragments, one register set per chunk pair of a step (SLAB2) or
    // two sets that the pairs alternate between (RING): A as MI x 8
    // consecutive k of a row; B as NJ x (two transpose reads of 4 consecutive
    // k of a column).
    constexpr int NSET = RINGS ? 2 : T::KP;
    u32x4 fa[NSET][MI];
    s16x4 fb[NSET][NJ][2];

    // Fragment read number o (0 .. NREAD - 1) of chunk pair kp of step kt, in
    // the order the matrix instructions first use them: A block 0, the NJ B
    // blocks (two transpose reads each), then A blocks 1 .. MI - 1.  Under
    // RING, h = kt & 1 picks the half of the A slab (a compile-time constant).
    auto read_piece = [&](int kt, int h, int kp, u32x4 (&a)[MI], s16x4 (&b)[NJ][2], int o) {
        if (o == 0 || o > 2 * NJ) {
            const int mi = o == 0 ? 0 : o - 2 * NJ;
            const int slab = RINGS ? (kt >> 1) : kt;
            const char* sa = smA + (slab % T::SA) * T::A_STAGE;
            a[mi] = *(const u32x4*)(sa + a16_off(wm * (TBM / 2) + mi * 32 + li,
                                                 (RINGS ? 4 * h : 0) + 2 * kp + g));
        } else {
            const char* sb = smB + (kt % T::SB) * T::B_STAGE;
            const int nj = (o - 1) >> 1, hh = (o - 1) & 1;
            const int k = kp * 16 + 8 * g + 4 * hh + ta;
            const int c = wn * (TBN / 16) + nj * 4 + 2 * tg + (tq >> 1);
            b[nj][hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
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
    // All reads of a pair, in the order the main loop issues them (the
    // compiler's wait counts at the loop's head are exact only if both paths
    // into it leave the reads in one order).
    auto read_frags = [&](int kt, int h, int kp, u32x4 (&a)[MI], s16x4 (&b)[NJ][2]) {
#pragma unroll
        for (int o = 0; o < T::NREAD; ++o) {
            read_piece(kt, h, kp, a, b, o);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Wait until at most VM of this wave's direct-to-LDS loads and LGKM of its
    // LDS accesses are in flight, then barrier.
    auto sync = [&](auto vm_tag, auto lgkm_tag) {
        constexpr int VM = decltype(vm_tag)::value;
        constexpr int LGKM = decltype(lgkm_tag)::value;
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(VM, LGKM));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    using AllLds = std::integral_constant<int, 0>;

    if constexpr (!RINGS) {
        // SLAB2, written out in issue order (sched_barrier pins it): with one
        // wave per SIMD nothing else hides a stall, so every load and LDS read
        // sits between two MFMAs.  Prologue: loads of steps 0 .. S - 1.  Step
        // kt: spread over the MFMAs of pairs 0 and 1, read the fragments of
        // pairs 1 .. KP - 1 (one register set per pair; each pair's reads are
        // issued before its MFMAs start); then wait until step kt + 1 has
        // landed (later steps may still be in flight) and barrier, which
        // retires every wave's reads of stage kt % S; then, spread over the
        // MFMAs of pairs 2 .. KP - 1, refill that stage with step kt + S and
        // read pair 0 of step kt + 1 (its stage landed before the barrier, and
        // pair 0's registers are free).  Spreading those reads over both pairs
        // rather than the last one measured 1-4 % faster on the tiles that are
        // not power-limited.  (A barrier after pair 0, with the refill over
        // three pairs, measured about 1 % slower.)  The last step reads that
        // pair too (from the stage the empty loads past K have zero-filled,
        // inside the LDS array; the registers are never used): an
        // unconditional read saves a branch per matrix instruction.
        using OneStepLeft = std::integral_constant<int, (T::SA - 1) * T::LOADS>;
        using TwoStepsLeft = std::integral_constant<int, (T::SA - 2) * T::LOADS>;
        if (nk > 0) {
#pragma unroll
            for (int s = 0; s < T::SA; ++s) {
                const LoadDesc d = load_desc(s, s);
#pragma unroll
                for (int j = 0; j < T::LOADS; ++j) dma_one(d, 0, j);
            }
            sync(OneStepLeft{}, AllLds{});
            if ((K % BKA) && nk == 1) { fix_tail(); sync(OneStepLeft{}, AllLds{}); }
            read_frags(0, 0, 0, fa[0], fb[0]);
            for (int kt = 0; kt < nk; ++kt) {
                constexpr int NR = T::NREAD * (T::KP - 1);
#pragma unroll
                for (int i = 0; i < 2 * T::NMFMA; ++i) {
                    if (i < T::NMFMA) mfma_one(fa[0], fb[0], i / NJ, snake(i));
                    else mfma_one(fa[1], fb[1], (i - T::NMFMA) / NJ, snake(i - T::NMFMA));
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int r = (i * NR) / (2 * T::NMFMA); r < ((i + 1) * NR) / (2 * T::NMFMA); ++r)
                        read_piece(kt, 0, 1 + r / T::NREAD, fa[1 + r / T::NREAD],
                                   fb[1 + r / T::NREAD], r % T::NREAD);
                    __builtin_amdgcn_sched_barrier(0);
                }
                // Every read of stage kt is now issued: retire them, wait for step
                // kt + 1, barrier.  The stage is then free for step kt + S.
                const LoadDesc d = load_desc(kt + T::SA, kt + T::SA);
                sync(TwoStepsLeft{}, AllLds{});
                if ((K % BKA) && kt + 2 == nk) { fix_tail(); sync(TwoStepsLeft{}, AllLds{}); }
                constexpr int SLOTS = T::NMFMA * (T::KP - 2);
#pragma unroll
                for (int kp = 2; kp < T::KP; ++kp) {
#pragma unroll
                    for (int i = 0; i < T::NMFMA; ++i) {
                        mfma_one(fa[kp], fb[kp], i / NJ, snake(i));
                        __builtin_amdgcn_sched_barrier(0);
                        const int slot = (kp - 2) * T::NMFMA + i;
#pragma unroll
                        for (int j = (slot * T::LOADS) / SLOTS; j < ((slot + 1) * T::LOADS) / SLOTS; ++j)
                            dma_one(d, 0, j);
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int r = (slot * T::NREAD) / SLOTS; r < ((slot + 1) * T::NREAD) / SLOTS; ++r)
                            read_piece(kt + 1, 0, 0, fa[0], fb[0], r);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
        }
    } else {
        // RING, written out in issue order like SLAB2.  Loads go out in step
        // order, LOADS per step (the prologue's first step has no B stage).
        // Before step 0's first read, A slab 0 and B stage 0 (the prologue's
        // first two steps) have landed.  At the top of step kt, everything
        // issued up to step kt - 2 (SA - 2) has landed: B stage kt + 1 was
        // issued in step kt + 2 - SB, and the slab holding step kt + 1 no later
        // than that.  LDS accesses complete in order, and the last NREAD a
        // wave issued before that barrier are its reads of pair 0 of step kt,
        // from a stage that is not refilled: only the older ones (the previous
        // step's) must be done before the barrier hands their slots (B stage
        // (kt - 1) % SB and, when kt is even, A slab ((kt >> 1) - 1) % SA) to
        // the loads.  Then the two chunk pairs of step kt: pair p's MFMAs carry
        // the reads of pair p + 1 (of step kt + 1 after the last pair) into the
        // other register set, in the order of first use, one read per MFMA from
        // the pair's first slot, so the last of them is several MFMAs old when
        // the next pair starts; and the step's loads are spread evenly over it.
        using StepZeroIn = std::integral_constant<int, (2 * T::SA - 4) * T::LOADS>;
        using NextStepIn = std::integral_constant<int, (2 * T::SA - 5) * T::LOADS>;
        using NextPairReads = std::integral_constant<int, T::NREAD>;
        constexpr int RSPAN = T::NREAD <= T::NMFMA ? T::NREAD : T::NMFMA;
        auto ring_desc = [&](int kt) { return load_desc((kt >> 1) + T::SA - 1, kt + T::SB - 1); };
        // TAIL: the step at whose top the last A slab has landed
        // (2 last_slab - 1) zeroes its K tail.  It is peeled off the main loop
        // so that the loop has no branch, whose join would otherwise make the
        // compiler wait for every LDS read before the step's first MFMA.
        auto step = [&](int kt, auto parity_tag, auto tail_tag) {
            constexpr int H = decltype(parity_tag)::value;     // kt & 1
            constexpr bool TAIL = decltype(tail_tag)::value;
            const LoadDesc d = ring_desc(kt);
            sync(NextStepIn{}, NextPairReads{});
            if constexpr (TAIL) { fix_tail(); sync(NextStepIn{}, AllLds{}); }
            constexpr int SLOTS = T::NMFMA * T::KP;
#pragma unroll
            for (int kp = 0; kp < T::KP; ++kp) {
#pragma unroll
                for (int i = 0; i < T::NMFMA; ++i) {
                    mfma_one(fa[kp & 1], fb[kp & 1], i / NJ, snake(i));
                    __builtin_amdgcn_sched_barrier(0);
                    const int slot = kp * T::NMFMA + i;
#pragma unroll
                    for (int j = (slot * T::LOADS) / SLOTS; j < ((slot + 1) * T::LOADS) / SLOTS; ++j)
                        dma_one(d, H, j);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int o = (i * T::NREAD) / RSPAN;
                         o < ((i + 1) * T::NREAD) / RSPAN && o < T::NREAD; ++o) {
                        if (kp + 1 < T::KP)
                            read_piece(kt, H, kp + 1, fa[(kp + 1) & 1], fb[(kp + 1) & 1], o);
                        else
                            read_piece(kt + 1, 1 - H, 0, fa[0], fb[0], o);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };
        using Even = std::integral_constant<int, 0>;
        using Odd = std::integral_constant<int, 1>;
        using NoTail = std::false_type;
        using Tail = std::true_type;
        if (nk > 0) {
            for (int kt = -(2 * T::SA - 2); kt < 0; kt += 2) {
                // Two prologue steps at a time (even, odd).  The first has no B
                // stage (its index would be -1): only its A loads go out, and
                // the wait counts only count loads issued after it.
                const LoadDesc d0 = ring_desc(kt);
                const int nload = kt + T::SB - 1 >= 0 ? T::LOADS : T::A_DMA;
                for (int j = 0; j < nload; ++j) dma_one(d0, 0, j);
                const LoadDesc d1 = ring_desc(kt + 1);
#pragma unroll
                for (int j = 0; j < T::LOADS; ++j) dma_one(d1, 1, j);
            }
            sync(StepZeroIn{}, AllLds{});
            // The step that zeroes the last slab's K tail is odd (or -1: before step 0).
            const int kt_fix = (K % BKA) ? 2 * last_slab - 1 : -2;
            if (kt_fix == -1) { fix_tail(); sync(StepZeroIn{}, AllLds{}); }
            read_frags(0, 0, 0, fa[0], fb[0]);
            int kt = 0;
            for (; kt + 1 < nk && kt + 1 != kt_fix; kt += 2) {
                step(kt, Even{}, NoTail{});
                step(kt + 1, Odd{}, NoTail{});
            }
            if (kt + 1 == kt_fix) {
                step(kt, Even{}, NoTail{});
                step(kt + 1, Odd{}, Tail{});
                kt += 2;
            }
            for (; kt + 1 < nk; kt += 2) {
                step(kt, Even{}, NoTail{});
                step(kt + 1, Odd{}, NoTail{});
            }
            if (kt < nk) step(kt, Even{}, NoTail{});
        }
    }
    // No direct-to-LDS write may still be in flight when the workgroup ends.
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
}

// One macro-tile per workgroup: tile map_tile(blockIdx.x), k range blockIdx.y.
template <int IN, int OUT, int TBM, int TBN, bool EPI, bool PAIRS, int SCHED, int S>
__global__ __launch_bounds__(256) void gemm16_kernel(
    const char* __restrict__ A, const char* __restrict__ B, char* __restrict__ C,
    int M, int N, int K, int lda, int ldb, int ldc, int tiles_m, int tiles_n,
    int kchunk, int64_t c_zstride, EpiArgs epi) {
    using T = Tile16<TBM, TBN, SCHED, S>;
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
    __shared__ __attribute__((aligned(1024))) char smem[T::LDS];
    int tm, tn;
    map_tile((int)blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * TBM;
    const int n0 = tn * TBN;
    const int rows_a = (M - m0) < TBM ? (M - m0) : TBM;
    const int cols_b = (N - n0) < TBN ? (N - n0) : TBN;
    f32x16 acc[T::MI][T::NJ];
    mainloop16<IN, TBM, TBN, SCHED, S>(A, B, K, lda, ldb, m0, n0, rows_a, cols_b, smem, acc);
    const int lane = (int)threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    store_tile<OUT, T::MI, T::NJ, EPI, PAIRS>(acc, C, M, N, ldc, m0 + (wave >> 1) * (TBM / 2),
                                              n0 + (wave & 1) * (TBN / 2), lane >> 5, lane & 31, epi);
}

// ------------------------------------------------------------------ Stream-K
//
// The schedule (which workgroup computes which k range of which tile, and
// which blocks of each tile it reduces) is in dgemm_internal.h, shared with
// the host-side query of it.  This kernel runs it: one persistent workgroup
// per CU, the 256 x 256 SLAB2 K loop for every piece.

using SkTile = Tile16<SK_TILE, SK_TILE, SLAB2, 2>;
constexpr int SK_SLOT = SK_TILE * SK_TILE * 4;  // bytes of one fp32 partial tile

// A partial tile in the accumulators' own layout: lane l of wave w keeps
// acc[mi][nj][4 c .. 4 c + 3] in 16-byte piece ((w MI NJ + mi NJ + nj) 4 + c) 64 + l
// of the slot, so every store and load instruction moves one contiguous KiB,
// and 32 x 32 output block q = w MI NJ + mi NJ + nj is the slot's KiB pieces
// 4 q .. 4 q + 3.
template <int MI, int NJ>
__device__ __forceinline__ void part_store(const f32x16 (&acc)[MI][NJ], char* slot, int wave,
                                           int lane) {
    f32x4* p = (f32x4*)slot + wave * (MI * NJ * 4 * 64) + lane;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                p[((mi * NJ + nj) * 4 + c) * 64] =
                    f32x4{acc[mi][nj][4 * c], acc[mi][nj][4 * c + 1], acc[mi][nj][4 * c + 2],
                          acc[mi][nj][4 * c + 3]};
}

constexpr int SK_BATCH = 8;  // contributors whose partials are loaded ahead of their additions

// This workgroup's share of tile u's reduction: blocks [lo, hi) of the tile,
// dealt to the four waves in turn.  Each output is the sum of the partials of
// the tile's contributors first .. last, added in that order, then the
// epilogue and the one-tile kernel's store of a 32 x 32 block (the
// accumulator layout the slot keeps).  Every partial is in its slot and
// visible to this workgroup.  A function of its own (arguments in registers),
// so that its registers are allocated apart from the K loop's.
template <int OUT, bool EPI, bool PAIRS>
__device__ __attribute__((noinline)) void sk_reduce(int x, int j, int W, int nk, int u, int tm,
                                                    int tn, const char* part, char* C, int M,
                                                    int N, int ldc, int wave, int lane,
                                                    float alpha, float beta, const float* bias,
                                                    int relu) {
    constexpr int MI = SkTile::MI, NJ = SkTile::NJ;
    SkRun r{};
    r.x = x;
    r.j = j;
    r.R = (int)gridDim.x / NUM_XCD;
    r.W = W;
    r.nk = nk;
    const EpiArgs e{alpha, beta, bias, relu};
    int lo, hi;
    sk_share(r, u, lo, hi);
    const int f = r.first(u), l = r.last(u);
    for (int q = lo + wave; q < hi; q += 4) {
        f32x4 s[4];
        for (int p0 = f; p0 <= l; p0 += SK_BATCH) {
            f32x4 v[SK_BATCH][4];
#pragma unroll
            for (int i = 0; i < SK_BATCH; ++i) {
                if (p0 + i > l) break;  // wave-uniform
                const f32x4* src =
                    (const f32x4*)(part + (int64_t)r.slot(p0 + i, u) * SK_SLOT) + q * 256 + lane;
#pragma unroll
                for (int c = 0; c < 4; ++c) v[i][c] = src[c * 64];
            }
#pragma unroll
            for (int i = 0; i < SK_BATCH; ++i)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    if (p0 + i == f) s[c] = v[i][c];
                    else if (p0 + i <= l) s[c] += v[i][c];
                }
        }
        f32x16 t[1][1];
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int k = 0; k < 4; ++k) t[0][0][4 * c + k] = s[c][k];
        const int w = q / (MI * NJ), mi = (q / NJ) % MI, nj = q % NJ;
        store_tile<OUT, 1, 1, EPI, PAIRS>(t, C, M, N, ldc,
                                          tm * SK_TILE + (w >> 1) * (SK_TILE / 2) + mi * 32,
                                          tn * SK_TILE + (w & 1) * (SK_TILE / 2) + nj * 32,
                                          lane >> 5, lane & 31, e);
    }
}

template <int IN, int OUT, bool EPI, bool PAIRS>
__global__ __launch_bounds__(256) void gemm16_sk_kernel(
    const char* __restrict__ A, const char* __restrict__ B, char* __restrict__ C, int M, int N,
    int K, int lda, int ldb, int ldc, SkSched sk, EpiArgs epi) {
    using T = SkTile;
    constexpr int MI = T::MI, NJ = T::NJ;
    __shared__ __attribute__((aligned(1024))) char smem[T::LDS];
    __shared__ int s_missing;
    const int G = (int)gridDim.x;
    const int tid = (int)threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // The first rank in [p, hi] other than `self` whose flag does not hold
    // this launch's epoch within wait_ticks (hi + 1 if none), polled by one
    // thread with plain atomic loads; one acquire then makes every published
    // piece visible to the workgroup.  Every wave gets the same answer.
    auto first_missing = [&](int x, int p, int hi, int self) {
        if (tid == 0) {
            const long long t_end = wall_clock64() + sk.wait_ticks;
            for (; p <= hi; ++p) {
                if (p == self) continue;
                const unsigned long long* f = sk.flags + (x + NUM_XCD * p);
                bool ok;
                for (;;) {
                    ok = __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == sk.epoch;
                    if (ok || wall_clock64() >= t_end) break;
                    __builtin_amdgcn_s_sleep(2);
                }
                if (!ok) break;
            }
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            s_missing = p;
        }
        __syncthreads();
        const int m = __builtin_amdgcn_readfirstlane(s_missing);
        __syncthreads();  // every wave has read s_missing before it is written again
        return m;
    };

    // Phase 0: this rank's pieces (pc counts them); then, for its first and
    // (if any) second tile, the pieces of the tile's other contributors that
    // are missing, computed here (cur: the next rank to check), and this
    // rank's share of the tile's reduction.  Only these counters live across
    // iterations; the run is derived again each time from an opaque copy of
    // the workgroup index, which keeps the loop's registers out of the K loop.
    int phase = 0, pc = 0, cur = -1;
    bool first_item = true;
    f32x16 acc[MI][NJ];
    for (;;) {
        int b = (int)blockIdx.x;
        asm volatile("" : "+s"(b));
        const SkRun r = sk_run(sk, b, G);
        int u, p;  // the piece to compute: rank p's range of tile u
        if (phase == 0) {
            if (pc < r.npieces) {
                u = r.u0 + pc;
                p = r.j;
                ++pc;
            } else {
                if (r.npieces == 0) break;
                // Publish: every wave's stores have completed, then the flag,
                // with release ordering.
                __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
                __syncthreads();
                if (tid == 0)
                    __hip_atomic_store(sk.flags + b, sk.epoch, __ATOMIC_RELEASE,
                                       __HIP_MEMORY_SCOPE_AGENT);
                phase = 1;
                cur = r.first(r.u0);
                continue;
            }
        } else {
            u = r.u0 + phase - 1;
            cur = first_missing(r.x, cur, r.last(u), r.j);
            if (cur > r.last(u)) {
                int tm, tn;
                map_tile(r.pos(u), sk.tiles_m, sk.tiles_n, tm, tn);
                sk_reduce<OUT, EPI, PAIRS>(r.x, r.j, r.W, r.nk, u, tm, tn, sk.part, C, M, N, ldc,
                                           wave, lane, epi.alpha, epi.beta, epi.bias, epi.relu);
                if (phase == r.npieces) break;
                ++phase;
                cur = r.first(r.u0 + 1);
                continue;
            }
            p = cur++;
        }
        if (!first_item) __syncthreads();  // every wave is done with the LDS ring and the slot
        first_item = false;

        int tm, tn, kb, ke;
        map_tile(r.pos(u), sk.tiles_m, sk.tiles_n, tm, tn);
        r.piece(p, u, kb, ke);
        const int m0 = tm * SK_TILE;
        const int n0 = tn * SK_TILE;
        const int rows_a = (M - m0) < SK_TILE ? (M - m0) : SK_TILE;
        const int cols_b = (N - n0) < SK_TILE ? (N - n0) : SK_TILE;
        const int kbeg = kb * SK_BK;
        const int kseg = (ke == r.nk ? K : ke * SK_BK) - kbeg;
        mainloop16<IN, SK_TILE, SK_TILE, SLAB2, 2, true, true>(
            A + (int64_t)kbeg * 2, B + (int64_t)kbeg * ldb * 2, kseg, lda, ldb, m0, n0, rows_a, cols_b,
            smem, acc);
        part_store<MI, NJ>(acc, sk.part + (int64_t)r.slot(p, u) * SK_SLOT, wave, lane);
        // A piece computed for another rank is read by this workgroup's waves
        // in the reduction: the barrier before it (in first_missing) orders them.
    }
}

template <int IN, int OUT, bool EPI, bool PAIRS>
hipError_t go_sk(const GemmLaunch& L, const SkSched& s, int grid) {
    const char* a = L.A;
    const char* b = L.B;
    char* c = L.C;
    int M = L.M, N = L.N, K = L.K, lda = L.lda, ldb = L.ldb, ldc = L.ldc;
    SkSched sk = s;
    EpiArgs e = L.e;
    void* args[] = {&a, &b, &c, &M, &N, &K, &lda, &ldb, &ldc, &sk, &e};
    return hipLaunchKernel((const void*)gemm16_sk_kernel<IN, OUT, EPI, PAIRS>, dim3((unsigned)grid),
                           dim3(256), args, 0, L.stream);
}

template <int IN, int OUT, bool EPI>
hipError_t sk_by_pairs(const GemmLaunch& L, const SkSched& s, int grid) {
    if (OUT != OUT_F32 && L.N % 2 == 0) return go_sk<IN, OUT, EPI, true>(L, s, grid);
    return go_sk<IN, OUT, EPI, false>(L, s, grid);
}

template <int IN, int OUT>
hipError_t sk_by_epi(const GemmLaunch& L, const SkSched& s, int grid) {
    return L.epi ? sk_by_pairs<IN, OUT, true>(L, s, grid) : sk_by_pairs<IN, OUT, false>(L, s, grid);
}

template <int IN, int OUT, int TBM, int TBN, bool EPI, bool PAIRS, int SCHED, int S>
hipError_t go(const GemmLaunch& L) {
    const char* a = L.A;
    const char* b = L.B;
    char* c = L.C;
    int M = L.M, N = L.N, K = L.K, lda = L.lda, ldb = L.ldb, ldc = L.ldc;
    int tiles_m = L.tiles_m, tiles_n = L.tiles_n, kchunk = L.kchunk;
    int64_t zs = L.c_zstride;
    EpiArgs e = L.e;
    void* args[] = {&a, &b, &c, &M, &N, &K, &lda, &ldb, &ldc, &tiles_m, &tiles_n, &kchunk, &zs, &e};
    return hipLaunchKernel((const void*)gemm16_kernel<IN, OUT, TBM, TBN, EPI, PAIRS, SCHED, S>,
                           dim3((unsigned)(tiles_m * tiles_n), (unsigned)L.splits), dim3(256),
                           args, 0, L.stream);
}

template <int IN, int OUT, bool EPI, bool PAIRS>
hipError_t by_tile(const GemmLaunch& L) {
    if (L.tbm == 256 && L.tbn == 256) return go<IN, OUT, 256, 256, EPI, PAIRS, SLAB2, 2>(L);
    if (L.tbm == 192 && L.tbn == 256) return go<IN, OUT, 192, 256, EPI, PAIRS, RING, 3>(L);
    if (L.tbm == 128 && L.tbn == 128)
        return L.stages == 4 ? go<IN, OUT, 128, 128, EPI, PAIRS, SLAB2, 4>(L)
                             : go<IN, OUT, 128, 128, EPI, PAIRS, SLAB2, 2>(L);
    return hipErrorInvalidValue;
}

// 16-bit C with an even N stores lane pairs; fp32 C, and 16-bit C with an odd
// N, one element per store.
template <int IN, int OUT, bool EPI>
hipError_t by_pairs(const GemmLaunch& L) {
    if (OUT != OUT_F32 && L.N % 2 == 0) return by_tile<IN, OUT, EPI, true>(L);
    return by_tile<IN, OUT, EPI, false>(L);
}

template <int IN, int OUT>
hipError_t by_epi(const GemmLaunch& L) {
    return L.epi ? by_pairs<IN, OUT, true>(L) : by_pairs<IN, OUT, false>(L);
}

}  // namespace

hipError_t launch_gemm16_sk(const GemmLaunch& L, const SkSched& s, int grid) {
    if (L.tbm != SK_TILE || L.tbn != SK_TILE || grid <= 0 || grid % NUM_XCD != 0 || s.nk <= 0)
        return hipErrorInvalidValue;
    if (L.in == IN_BF16) {
        if (L.out == OUT_F32) return sk_by_epi<IN_BF16, OUT_F32>(L, s, grid);
        if (L.out == OUT_BF16) return sk_by_epi<IN_BF16, OUT_BF16>(L, s, grid);
    } else if (L.in == IN_F16) {
        if (L.out == OUT_F32) return sk_by_epi<IN_F16, OUT_F32>(L, s, grid);
        if (L.out == OUT_F16) return sk_by_epi<IN_F16, OUT_F16>(L, s, grid);
    }
    return hipErrorInvalidValue;
}

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
