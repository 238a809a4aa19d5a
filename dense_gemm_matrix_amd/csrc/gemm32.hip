// gemm32.hip -- GEMM kernels for fp32 inputs on gfx950 (MI355X).
//
//   * gemm32_kernel: gfx950 has no reduced-precision (xf32) matrix
//     instruction, so products use full-precision v_mfma_f32_32x32x2_f32.
//     Operands go straight from global memory into a double-buffered LDS
//     ring (BK = 32) with direct-to-LDS loads; B stays N-contiguous there.
//   * gemm32x3_kernel: the same data on bf16 matrix instructions, each input
//     split in two bf16 parts and three products taken per term.
//
// Both are templates over a square macro-tile of 256 or 128 (128 x 128 uses
// 64 KiB of LDS, so two workgroups share a CU); the fp32 kernel is launched
// at 128 only, which measured faster at every shape.  Workgroup layout, tile map,
// swizzle principle, edge handling and epilogue as in the 16-bit kernel: 4
// waves in a 2 x 2 layout, each wave (TB/2)^2 as blocks of 32 x 32 fp32
// accumulators.

#include <type_traits>

#include "kern_common.h"

namespace dgemm {
namespace {
constexpr int BK = 32;                        // K per step (fp32: 128-byte LDS rows)

// Split-K: workgroup row z of the grid covers k in [z kchunk, (z+1) kchunk)
// and writes its partial sums at C + z c_zstride (z = 0, kchunk = K when
// unsplit).  Shifts the operand bases and narrows K to the window.
__device__ __forceinline__ void split_k_window(const char* __restrict__& A,
                                               const char* __restrict__& B,
                                               char* __restrict__& C, int& K,
                                               int ldb, int kchunk, int64_t c_zstride) {
    const int z = (int)blockIdx.y;
    const int kbeg = z * kchunk;
    A += (int64_t)kbeg * 4;
    B += (int64_t)kbeg * ldb * 4;
    C += z * c_zstride;
    K = (K - kbeg) < kchunk ? (K - kbeg) : kchunk;
}

constexpr int ROW_CHUNKS32 = 8;                  // 16-byte chunks per staged row (32 fp32)

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

// Square TB x TB macro-tile (256 or 128), 4 waves in a 2 x 2 layout, each wave
// (TB/2)^2 = MI x MI blocks of 32 x 32 accumulators.  Both operands go from
// global memory straight into LDS (direct-to-LDS buffer loads, 16 bytes per
// lane, lane-linear in LDS), NA = TB / 32 loads of A and as many of B per wave
// and step:
//   * A, K-contiguous as in memory: load i of wave w fills rows 8 (w NA + i) ..
//     + 7 (eight 16-byte chunks per row), lane l taking the global chunk that
//     belongs in slot l % 8 under lds32_index's swizzle; read with
//     ds_read_b128, four k of one row per lane.
//   * B, N-contiguous as in memory (TB / 4 chunks per k-row): load i of wave w
//     fills k-rows ROWB (w NA + i) .. + ROWB - 1; the chunk slots of k-rows
//     with bit 2 set are rotated by 8 (32 fp32), so that the two lane halves of
//     a fragment read, k-rows 4 apart, fall in different LDS banks.  A lane
//     needs four k of one column: two ds_read2st64_b32, each two k-rows apart
//     by one row pitch.
// Where the operands used to pass through registers (B transposed there, then
// written to LDS), the step now issues no LDS stores, and 4096^3 measured 4 %
// faster (980 against 1021 us, bitwise the same results).
template <bool EPI, int TB>
__global__ __launch_bounds__(NTHREADS) void gemm32_kernel(
    const char* __restrict__ A, const char* __restrict__ B, char* __restrict__ C,
    int M, int N, int K, int lda, int ldb, int ldc, int tiles_m, int tiles_n,
    int kchunk, int64_t c_zstride, EpiArgs epi) {
    static_assert(TB == 256 || TB == 128, "tile");
    constexpr int MI = TB / 64;               // 32 x 32 blocks per wave per dimension
    constexpr int NA = TB / 32;               // loads of A (and of B) per wave per step
    constexpr int BCH = TB / 4;               // 16-byte chunks per B k-row
    constexpr int ROWB = 64 / BCH;            // B k-rows per load
    constexpr int STAGE_CHUNKS = TB * ROW_CHUNKS32;
    split_k_window(A, B, C, K, ldb, kchunk, c_zstride);
    // [stage][operand: 0 = A, 1 = B][chunk]: 2 x 2 x (TB / 8) KiB.
    __shared__ u32x4 lds[2][2][STAGE_CHUNKS];

    int tm, tn;
    map_tile((int)blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int tid = (int)threadIdx.x;
    const int lane = tid & 63;
    // wave-uniform: the loads' LDS addresses go through M0
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m0 = tm * TB;
    const int n0 = tn * TB;
    const int rows_a = (M - m0) < TB ? (M - m0) : TB;
    const int cols_b = (N - n0) < TB ? (N - n0) : TB;
    const int nk = (K + BK - 1) / BK;
    const bool ragged_k = (K % BK) != 0;

    // Global byte offsets of this lane's loads within a step's resources.
    int voff_a[NA], voff_b[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        const int row = (wave * NA + i) * 8 + lane / 8;
        const int c = (lane & 7) ^ ((row ^ (row >> 3)) & 7);
        voff_a[i] = row * lda * 4 + c * 16;
        const int k = (wave * NA + i) * ROWB + lane / BCH;
        const int cb = (lane % BCH - ((k >> 2) & 1) * 8 + BCH) % BCH;
        voff_b[i] = k * ldb * 4 + cb * 16;
    }

    // Global loads of step kt into LDS stage s: step_desc makes the two
    // resources, load_one issues load j (0 .. NLOAD - 1, A's first) so that the
    // main loop can spread them over matrix instructions.
    constexpr int NLOAD = 2 * NA;
    struct StepDesc {
        __amdgpu_buffer_rsrc_t a, b;
    };
    auto step_desc = [&](int kt) {  // steps at or past the end: empty ranges (zeros)
        const int k0 = kt * BK;
        const int krem = K - k0;
        const char* abase = A + ((int64_t)m0 * lda + k0) * 4;
        const int64_t abytes = krem > 0 ? ((int64_t)(rows_a - 1) * lda + krem) * 4 : 0;
        const int rows_b = krem < BK ? krem : BK;
        const char* bbase = B + ((int64_t)k0 * ldb + n0) * 4;
        const int64_t bbytes = rows_b > 0 ? ((int64_t)(rows_b - 1) * ldb + cols_b) * 4 : 0;
        return StepDesc{make_rsrc(abase, abytes), make_rsrc(bbase, bbytes)};
    };
    auto load_one = [&](const StepDesc& d, int j, int s) {
        if (j < NA)
            dma16(d.a, lds_addr((const char*)&lds[s][0][0]) + (wave * NA + j) * 1024, voff_a[j]);
        else
            dma16(d.b, lds_addr((const char*)&lds[s][1][0]) + (wave * NA + j - NA) * 1024,
                  voff_b[j - NA]);
    };
    // The last step of a ragged K: A's columns at or past K hold other data
    // (row padding or the next row; B's k-rows past K read as zeros), zeroed in
    // LDS so that 0 * (NaN or Inf) cannot reach a sum.  Each lane fixes the
    // chunks its own loads wrote, after waiting for them.
    auto fix_tail = [&](int kt, int s) {
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            const int row = (wave * NA + i) * 8 + lane / 8;
            const int c = (lane & 7) ^ ((row ^ (row >> 3)) & 7);
            u32x4& v = lds[s][0][(wave * NA + i) * 64 + lane];
            v = mask_tail32(v, K - kt * BK - c * 4);
        }
    };

    const int wm = wave >> 1;
    const int wn = wave & 1;
    const int g = lane >> 5;   // lane group: which 4 k of a chunk pair
    const int li = lane & 31;  // row of A / column of B within a 32-block

    f32x16 acc[MI][MI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int nj = 0; nj < MI; ++nj)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][nj][r] = 0.0f;

    // Operand fragments for one chunk pair (8 k): lane group g holds k 8 kp + 4 g
    // .. + 3 of its MI A rows and MI B columns.  Two register sets alternate so
    // that the reads for pair kp + 1 are in flight while kp computes.
    u32x4 fa[2][MI], fb[2][MI];

    auto read_frags = [&](int s, int kp, u32x4 (&a)[MI], u32x4 (&b)[MI]) {
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
            a[mi] = lds[s][0][lds32_index(wm * (TB / 2) + mi * 32 + li, 2 * kp + g)];
#pragma unroll
        for (int nj = 0; nj < MI; ++nj) {
            const int n = wn * (TB / 2) + nj * 32 + li;
            const float* bp = (const float*)&lds[s][1][0] + (8 * kp + 4 * g) * TB +
                              ((n / 4 + 8 * g) % BCH) * 4 + (n & 3);
            b[nj] = u32x4{__builtin_bit_cast(uint32_t, bp[0]), __builtin_bit_cast(uint32_t, bp[TB]),
                          __builtin_bit_cast(uint32_t, bp[2 * TB]),
                          __builtin_bit_cast(uint32_t, bp[3 * TB])};
        }
    };

    // The MI x MI x 4 matrix instructions of one chunk pair (k-quarter e
    // outermost, so consecutive ones use different accumulators); after
    // instruction i, `after(i)` issues whatever the schedule places there.
    constexpr int NMP = MI * MI * 4;
    auto mfma_frags = [&](const u32x4 (&a)[MI], const u32x4 (&b)[MI], auto&& after) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int nj = 0; nj < MI; ++nj) {
                    acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                        as_float(a[mi][e]), as_float(b[nj][e]), acc[mi][nj], 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                    after((e * MI + mi) * MI + nj);
                    __builtin_amdgcn_sched_barrier(0);
                }
    };
    auto nothing = [](int) {};

    // Schedule of one K step (stage `cur` in LDS, stage cur ^ 1 being filled),
    // in issue order: read pair 1; pair 0's matrix instructions, with the loads
    // of step kt + 1 into stage cur ^ 1 spread among them (that stage's last
    // reads were retired before the previous barrier); read pair 2; pair 1;
    // read pair 3; pair 2; wait for this wave's loads, barrier; read pair 0 of
    // stage cur ^ 1; pair 3 (already in registers), which covers that read's
    // latency.  The loads are inline assembly the compiler does not count, so
    // the waits before each barrier are explicit.  sched_barrier keeps the
    // compiler from sinking the fragment reads down to their uses and from
    // gathering the loads into a block, which would stall the matrix pipe.
    if (nk > 0) {
        {
            const StepDesc d0 = step_desc(0);
#pragma unroll
            for (int j = 0; j < NLOAD; ++j) load_one(d0, j, 0);
            if (ragged_k && nk == 1) fix_tail(0, 0);
        }
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));
        __syncthreads();
        read_frags(0, 0, fa[0], fb[0]);
        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            const bool more = kt + 1 < nk;
            const StepDesc nd = step_desc(kt + 1);
            read_frags(cur, 1, fa[1], fb[1]);
            __builtin_amdgcn_sched_barrier(0);
            mfma_frags(fa[0], fb[0], [&](int i) {
#pragma unroll
                for (int j = (i * NLOAD) / NMP; j < ((i + 1) * NLOAD) / NMP; ++j) load_one(nd, j, cur ^ 1);
            });
            __builtin_amdgcn_sched_barrier(0);
            read_frags(cur, 2, fa[0], fb[0]);
            __builtin_amdgcn_sched_barrier(0);
            mfma_frags(fa[1], fb[1], nothing);
            __builtin_amdgcn_sched_barrier(0);
            read_frags(cur, 3, fa[1], fb[1]);
            __builtin_amdgcn_sched_barrier(0);
            if (ragged_k && kt + 2 == nk) fix_tail(kt + 1, cur ^ 1);
            __builtin_amdgcn_sched_barrier(0);
            mfma_frags(fa[0], fb[0], nothing);
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));
            __syncthreads();
            if (more) read_frags(cur ^ 1, 0, fa[0], fb[0]);
            __builtin_amdgcn_sched_barrier(0);
            mfma_frags(fa[1], fb[1], nothing);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    store_tile<OUT_F32, MI, MI, EPI, false>(acc, C, M, N, ldc, m0 + wm * (TB / 2), n0 + wn * (TB / 2), g,
                                     li, epi);
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

constexpr int X3_ROW = BK * 2;                  // 64-byte bf16 rows: 4 chunks of 8 k

// Byte offset of chunk c (0..3) of bf16 row r in one part of a stage.  Four
// 64-byte rows span the 256 bytes of LDS banks, so rows r and r + 4 share
// banks.  B's transposing stores write rows 4 apart from neighbouring lanes
// (16 rows per 64-lane store); the fragment reads take 4 consecutive rows at
// one chunk per group of 4 lanes.  Rows are therefore permuted inside each
// group of four (slot (r ^ r >> 2) & 3) and chunks XORed with (r >> 2) & 3:
// the reads still see 4 rows in 4 distinct quarters of the banks, and rows
// 4 apart now land in different quarters and chunk positions, so 8- and
// 16-lane groups of either store touch distinct 16-byte bank groups.
__device__ __forceinline__ int x3_off(int row, int chunk) {
    const int slot = (row & ~3) | ((row ^ (row >> 2)) & 3);
    return slot * X3_ROW + ((chunk ^ ((row >> 2) & 3)) << 4);
}

// Split two fp32 values into packed hi and lo bf16 parts (x0 in the low half
// of each word).  One two-wide conversion per part (v_cvt_pk_bf16_f32, nearest
// even); hi widens back to fp32 exactly by placing its bits in the upper half
// of a word.  Six VALU instructions.
__device__ __forceinline__ void split_pair(float x0, float x1, uint32_t& hi, uint32_t& lo) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const f32x2 v = {x0, x1};
    const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
    const f32x2 hf = {as_float(h << 16), as_float(h & 0xffff0000u)};
    hi = h;
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(v - hf, bf16x2));
}

// Split eight fp32 values (x, then y) into packed bf16 hi and lo parts, value
// j in half j % 2 of word j / 2.
__device__ __forceinline__ void split8(u32x4 x, u32x4 y, u32x4& hi, u32x4& lo) {
    uint32_t h[4], l[4];
    split_pair(as_float(x[0]), as_float(x[1]), h[0], l[0]);
    split_pair(as_float(x[2]), as_float(x[3]), h[1], l[1]);
    split_pair(as_float(y[0]), as_float(y[1]), h[2], l[2]);
    split_pair(as_float(y[2]), as_float(y[3]), h[3], l[3]);
    hi = u32x4{h[0], h[1], h[2], h[3]};
    lo = u32x4{l[0], l[1], l[2], l[3]};
}

// Square TB x TB macro-tile (256 or 128), 4 waves in a 2 x 2 layout, each
// wave (TB/2)^2 = MI x MI blocks of 32 x 32 accumulators.  Staging per step
// (BK = 32): A is TB rows, thread -> 8 consecutive k (two 16-byte fp32
// pieces) of rows ar0 + 64 i (i < TB / 64); B is 32 k-rows x TB columns,
// thread -> a KB k x 4 column block, KB = 8 at TB = 256 and 4 at TB = 128 (256
// blocks either way).
template <bool EPI, int TB>
__global__ __launch_bounds__(NTHREADS) void gemm32x3_kernel(
    const char* __restrict__ A, const char* __restrict__ B, char* __restrict__ C,
    int M, int N, int K, int lda, int ldb, int ldc, int tiles_m, int tiles_n,
    int kchunk, int64_t c_zstride, EpiArgs epi) {
    static_assert(TB == 256 || TB == 128, "tile");
    constexpr int MI = TB / 64;                  // 32 x 32 blocks per wave per dimension
    constexpr int AR = TB / 64;                  // A rows per thread per step
    constexpr int KB = TB == 256 ? 8 : 4;        // B k-rows per thread block
    constexpr int PART = TB * X3_ROW;            // one part of one operand
    constexpr int STAGE = 4 * PART;              // A hi, A lo, B hi, B lo
    constexpr int NU = AR + 4;                   // store units per step
    constexpr int NM = MI * MI * 3;              // MFMAs per chunk pair
    constexpr int NR = 4 * MI;                   // fragment reads per chunk pair
    split_k_window(A, B, C, K, ldb, kchunk, c_zstride);
    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

    int tm, tn;
    map_tile((int)blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int tid = (int)threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int m0 = tm * TB;
    const int n0 = tn * TB;
    const int rows_a = (M - m0) < TB ? (M - m0) : TB;
    const int cols_b = (N - n0) < TB ? (N - n0) : TB;
    const int nk = (K + BK - 1) / BK;
    const bool ragged_k = (K % BK) != 0;

    const int ac = tid & 3;
    const int ar0 = tid >> 2;
    const int kb = tid % (BK / KB);
    const int nb = tid / (BK / KB);

    int voff_a[AR], voff_b[KB];
#pragma unroll
    for (int i = 0; i < AR; ++i) voff_a[i] = (ar0 + 64 * i) * lda * 4 + ac * 32;
#pragma unroll
    for (int i = 0; i < KB; ++i) voff_b[i] = (kb * KB + i) * ldb * 4 + nb * 16;

    // Staging registers: one set at 256 x 256 (the register file is full), two
    // at 128 x 128, where step kt's loads fetch step kt + 3 into the set that
    // step kt + 1's pieces have just emptied, three chunk pairs ahead of their
    // use instead of one (a grid of one workgroup per CU has nothing else to
    // hide that latency).  Set indices are compile-time: I0 / I1 below.
    constexpr int NSET = TB == 128 ? 2 : 1;
    u32x4 ra[NSET][2 * AR], rb[NSET][KB];
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1 % NSET>;

    // Global loads of step kt into registers.  Steps at or past the end get
    // empty ranges and load zeros (the schedule below issues them
    // unconditionally; their data is never used).  On the last step of a
    // ragged K, A's columns at or past K hold other data (row padding or the
    // next row) and are zeroed (mask_a), since the matching B rows are zero;
    // that waits for the loads, once per call.  step_desc makes the step's two
    // resources; load_one issues load j (0 .. NLOAD - 1, A's first), so that
    // the main loop can spread them over matrix instructions.
    constexpr int NLOAD = 2 * AR + KB;
    struct StepDesc {
        __amdgpu_buffer_rsrc_t a, b;
    };
    auto step_desc = [&](int kt) {
        const int k0 = kt * BK;
        const int krem = K - k0;
        const char* abase = A + ((int64_t)m0 * lda + k0) * 4;
        const int64_t abytes = krem > 0 ? ((int64_t)(rows_a - 1) * lda + krem) * 4 : 0;
        const int rows_b = krem < BK ? krem : BK;
        const char* bbase = B + ((int64_t)k0 * ldb + n0) * 4;
        const int64_t bbytes = rows_b > 0 ? ((int64_t)(rows_b - 1) * ldb + cols_b) * 4 : 0;
        return StepDesc{make_rsrc(abase, abytes), make_rsrc(bbase, bbytes)};
    };
    auto load_one = [&](const StepDesc& d, int j, auto set) {
        constexpr int P = decltype(set)::value;
        if (j < 2 * AR)
            ra[P][j] = load16(d.a, voff_a[j >> 1] + (j & 1) * 16);
        else
            rb[P][j - 2 * AR] = load16(d.b, voff_b[j - 2 * AR]);
    };
    auto mask_a = [&](int kt, auto set) {
        constexpr int P = decltype(set)::value;
        const int valid = K - kt * BK - ac * 8;
#pragma unroll
        for (int i = 0; i < AR; ++i) {
            ra[P][2 * i] = mask_tail32(ra[P][2 * i], valid);
            ra[P][2 * i + 1] = mask_tail32(ra[P][2 * i + 1], valid - 4);
        }
    };
    auto load_step = [&](int kt, bool tail, auto set) {
        const StepDesc d = step_desc(kt);
#pragma unroll
        for (int j = 0; j < NLOAD; ++j) load_one(d, j, set);
        if (tail) mask_a(kt, set);
    };

    // Store unit u (0 .. NU - 1) into stage s: u < AR splits A row ar0 + 64 u
    // (8 k: one chunk per part); u >= AR splits column u - AR of the B block
    // (KB k: one chunk per part at KB = 8, half a chunk at KB = 4).  A unit is
    // done in pieces so that its work can be spread over several matrix
    // instructions: piece w < unit_pairs(u) splits value pair w into uh[w],
    // ul[w]; the last piece writes both parts to LDS.
    uint32_t uh[4], ul[4];
    auto unit_pairs = [](int u) { return u < AR ? 4 : KB / 2; };
    auto unit_piece = [&](int s, int u, int w, auto set) __attribute__((always_inline)) {
        constexpr int P = decltype(set)::value;
        if (w < unit_pairs(u)) {
            float x0, x1;
            if (u < AR) {
                const u32x4& r = ra[P][2 * u + (w >> 1)];
                x0 = as_float(r[(w & 1) * 2]);
                x1 = as_float(r[(w & 1) * 2 + 1]);
            } else {
                x0 = as_float(rb[P][2 * w][u - AR]);
                x1 = as_float(rb[P][2 * w + 1][u - AR]);
            }
            // Empty volatile asm statements pin the split to this point of the
            // schedule: the instruction selector orders them with the
            // sched_barriers, which pure arithmetic alone does not follow.
            asm volatile("" : "+v"(x0), "+v"(x1));
            split_pair(x0, x1, uh[w], ul[w]);
            asm volatile("" ::"v"(uh[w]), "v"(ul[w]));
            return;
        }
        char* st = smem + s * STAGE;
        if (u < AR) {
            const int off = x3_off(ar0 + 64 * u, ac);
            *(u32x4*)(st + off) = u32x4{uh[0], uh[1], uh[2], uh[3]};
            *(u32x4*)(st + PART + off) = u32x4{ul[0], ul[1], ul[2], ul[3]};
        } else {
            const int cc = u - AR;
            char* base = st + 2 * PART;
            if constexpr (KB == 8) {
                const int off = x3_off(nb * 4 + cc, kb);
                *(u32x4*)(base + off) = u32x4{uh[0], uh[1], uh[2], uh[3]};
                *(u32x4*)(base + PART + off) = u32x4{ul[0], ul[1], ul[2], ul[3]};
            } else {
                typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
                const int off = x3_off(nb * 4 + cc, kb >> 1) + (kb & 1) * 8;
                *(u32x2*)(base + off) = u32x2{uh[0], uh[1]};
                *(u32x2*)(base + PART + off) = u32x2{ul[0], ul[1]};
            }
        }
    };
    // Pieces in order: unit 0's pairs and write, unit 1's, ...
    constexpr int NPIECE = AR * 5 + 4 * (KB / 2 + 1);
    auto store_pieces = [&](int s, int p0, int p1, auto set) __attribute__((always_inline)) {  // pieces [p0, p1)
#pragma unroll
        for (int p = p0; p < p1; ++p) {
            constexpr int PB = KB / 2 + 1;  // pieces per B unit
            if (p < AR * 5)
                unit_piece(s, p / 5, p % 5, set);
            else
                unit_piece(s, AR + (p - AR * 5) / PB, (p - AR * 5) % PB, set);
        }
    };
    auto store_unit = [&](int s, int u, auto set) __attribute__((always_inline)) {
#pragma unroll
        for (int w = 0; w <= unit_pairs(u); ++w) unit_piece(s, u, w, set);
    };

    const int wm = wave >> 1;
    const int wn = wave & 1;
    const int g = lane >> 5;
    const int li = lane & 31;

    f32x16 acc[MI][MI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int nj = 0; nj < MI; ++nj)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][nj][r] = 0.0f;

    // Fragments of one 16-k chunk pair: [part][block], part 0 = hi, 1 = lo.
    u32x4 fa[2][2][MI], fb[2][2][MI];

    // Fragment read r (0 .. NR - 1) of pair kp from stage s: part r / (2 MI);
    // A block q = r % (2 MI) when q < MI, else B block q - MI.
    auto read_one = [&](int s, int kp, u32x4 (&a)[2][MI], u32x4 (&b)[2][MI], int r) {
        const char* st = smem + s * STAGE;
        const int ch = 2 * kp + g;
        const int p = r / (2 * MI), q = r % (2 * MI);
        if (q < MI)
            a[p][q] = *(const u32x4*)(st + p * PART + x3_off(wm * (TB / 2) + q * 32 + li, ch));
        else
            b[p][q - MI] =
                *(const u32x4*)(st + (2 + p) * PART + x3_off(wn * (TB / 2) + (q - MI) * 32 + li, ch));
    };

    // Matrix instruction i (0 .. NM - 1) of a pair: block i / 3 (mi, nj),
    // product i % 3: the small terms first, then the leading one.
    auto mfma_one = [&](const u32x4 (&a)[2][MI], const u32x4 (&b)[2][MI], int i) {
        const int mi = (i / 3) / MI, nj = (i / 3) % MI, t = i % 3;
        const u32x4 av = t == 0 ? a[1][mi] : a[0][mi];
        const u32x4 bv = t == 1 ? b[1][nj] : b[0][nj];
        acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv), acc[mi][nj], 0, 0, 0);
    };

    // Schedule of step kt (stage cur holds it, stage cur ^ 1 receives step
    // kt + 1), in issue order; sched_barrier pins it:
    //   pair 0's first NM / 2 MFMAs, carrying the NR reads of pair 1;
    //   from the middle of pair 0 to the middle of pair 1 (NM MFMA slots), the
    //   NPIECE store pieces of step kt + 1 (A rows, then B columns), spread
    //   evenly: at 256 x 256 at most one per slot, six VALU instructions or two
    //   LDS writes, few enough to issue while the matrix instruction before
    //   them runs; pair 1's first half also carries the 2 AR global loads of
    //   step kt + 2's A (the A pieces have emptied those registers);
    //   barrier (stage cur ^ 1 complete; every read of stage cur issued);
    //   pair 1's second half, carrying the NR reads of step kt + 1's pair 0 and
    //   the KB loads of step kt + 2's B (the B pieces have emptied those).
    // Every load is thus issued about NM slots before its first use, and no
    // slot carries more than two memory instructions.  With two staging sets
    // (128 x 128) the same slots load step kt + 3 into the set step kt + 1's
    // pieces have just emptied, 2 NM slots earlier than one set allows: 6-12 %
    // faster on grids of one workgroup per CU (2048^3: 65.5 -> 61.3 us,
    // 1536 x 1536 x 6144: 179.8 -> 158.8 us), the same results bit for bit.  The last steps also
    // load, split and store steps nk and nk + 1 (empty ranges: zeros, inside
    // the LDS array; never read).
    auto pieces_at = [&](int s, int slot, auto set) __attribute__((always_inline)) {  // the pieces placed after MFMA slot (0 .. 2 NM - 1)
        const int d = slot - NM / 2;
        if (d >= 0 && d < NM) store_pieces(s, (d * NPIECE) / NM, ((d + 1) * NPIECE) / NM, set);
    };
    // One step; `set` holds step kt + 1's loaded values, which this step splits
    // into stage cur ^ 1, and then receives the loads of step kt + 1 + NSET.
    auto step = [&](int kt, auto set) __attribute__((always_inline)) {
        const int cur = kt & 1;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            mfma_one(fa[0], fb[0], i);
            __builtin_amdgcn_sched_barrier(0);
            constexpr int Q = NM / 2;  // the slots before the first store piece
            if (i < Q) {
#pragma unroll
                for (int r = (i * NR) / Q; r < ((i + 1) * NR) / Q; ++r)
                    read_one(cur, 1, fa[1], fb[1], r);
            }
            if (i == NM / 2 - 1 && ragged_k && kt + 2 == nk) mask_a(kt + 1, set);
            pieces_at(cur ^ 1, i, set);
            __builtin_amdgcn_sched_barrier(0);
        }
        // Step kt + 1 + NSET's loads: A's into the registers the A pieces have
        // just emptied, B's after the barrier.
        const StepDesc nd = step_desc(kt + 1 + NSET);
        constexpr int H = NM - NM / 2;
#pragma unroll
        for (int i = 0; i < NM / 2; ++i) {
            mfma_one(fa[1], fb[1], i);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int l = (i * 2 * AR) / H; l < ((i + 1) * 2 * AR) / H; ++l) load_one(nd, l, set);
            pieces_at(cur ^ 1, NM + i, set);
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
#pragma unroll
        for (int i = NM / 2; i < NM; ++i) {
            mfma_one(fa[1], fb[1], i);
            __builtin_amdgcn_sched_barrier(0);
            const int j = i - NM / 2;
#pragma unroll
            for (int l = (j * KB) / H; l < ((j + 1) * KB) / H; ++l) load_one(nd, 2 * AR + l, set);
#pragma unroll
            for (int r = (j * NR) / H; r < ((j + 1) * NR) / H; ++r)
                read_one(cur ^ 1, 0, fa[0], fb[0], r);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if (nk > 0) {
        load_step(0, ragged_k && nk == 1, I0{});
#pragma unroll
        for (int u = 0; u < NU; ++u) store_unit(0, u, I0{});
        __syncthreads();
#pragma unroll
        for (int r = 0; r < NR; ++r) read_one(0, 0, fa[0], fb[0], r);
        // Later steps' tail masks, if any, are applied in the loop.
        load_step(1, false, I1{});
        if constexpr (NSET == 2) {
            load_step(2, false, I0{});
            for (int kt = 0; kt < nk; kt += 2) {
                step(kt, I1{});
                if (kt + 1 < nk) step(kt + 1, I0{});
            }
        } else {
            // One set (256 x 256): the same schedule written as a plain loop,
            // which keeps the compiler's code for this instantiation as it was.
            for (int kt = 0; kt < nk; ++kt) {
                const int cur = kt & 1;
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < NM; ++i) {
                    mfma_one(fa[0], fb[0], i);
                    __builtin_amdgcn_sched_barrier(0);
                    constexpr int Q = NM / 2;
                    if (i < Q) {
#pragma unroll
                        for (int r = (i * NR) / Q; r < ((i + 1) * NR) / Q; ++r)
                            read_one(cur, 1, fa[1], fb[1], r);
                    }
                    if (i == NM / 2 - 1 && ragged_k && kt + 2 == nk) mask_a(kt + 1, I0{});
                    pieces_at(cur ^ 1, i, I0{});
                    __builtin_amdgcn_sched_barrier(0);
                }
                const StepDesc nd = step_desc(kt + 2);
                constexpr int H = NM - NM / 2;
#pragma unroll
                for (int i = 0; i < NM / 2; ++i) {
                    mfma_one(fa[1], fb[1], i);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int l = (i * 2 * AR) / H; l < ((i + 1) * 2 * AR) / H; ++l) load_one(nd, l, I0{});
                    pieces_at(cur ^ 1, NM + i, I0{});
                    __builtin_amdgcn_sched_barrier(0);
                }
                __syncthreads();
#pragma unroll
                for (int i = NM / 2; i < NM; ++i) {
                    mfma_one(fa[1], fb[1], i);
                    __builtin_amdgcn_sched_barrier(0);
                    const int j = i - NM / 2;
#pragma unroll
                    for (int l = (j * KB) / H; l < ((j + 1) * KB) / H; ++l) load_one(nd, 2 * AR + l, I0{});
#pragma unroll
                    for (int r = (j * NR) / H; r < ((j + 1) * NR) / H; ++r)
                        read_one(cur ^ 1, 0, fa[0], fb[0], r);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    }

    store_tile<OUT_F32, MI, MI, EPI, false>(acc, C, M, N, ldc, m0 + wm * (TB / 2), n0 + wn * (TB / 2), g,
                                     li, epi);
}

// ---------------------------------------------------------------- fp32, K sliced over the waves
//
// For products whose output is too small to give every CU a 128 x 128 tile
// (512^3 has 16 of them for 256 CUs), the parallelism that split-K finds in K
// (the nine-levels tutorial, section 2.9) is found inside the workgroup
// instead: a workgroup of W waves owns a small TS x TS tile (TS = 32 MI), and
// its waves split K between them, each an equal run of 32-k blocks, so that
// every wave holds the whole tile's accumulators for its own k.  The W partial
// tiles are then added through LDS in wave order, each wave summing and storing
// (with the fused epilogue) an equal share of the tile: no partial sums leave
// the CU, no workspace is needed and no second kernel runs.
//
// No operand is shared between the waves, so each wave moves its own.  For
// unit u of a block (8 k):
//   * A: lane (g, li) fetches k = 8u + 4g .. 8u + 4g + 3 of A's row li as one
//     16-byte load into registers.
//   * B at TS = 32: lane (g, li) fetches its column's element at each of
//     those k with a 4-byte load (each half-wave reads 128 contiguous bytes of
//     a B row), 16 per block.
//   * B at TS = 64 (BL): 32 such loads per block would keep the CU's texture
//     addresser, which costs the same per load instruction whatever its width,
//     busier than the matrix work; the block's 32 k-rows x 64 columns go
//     instead into the wave's own LDS region as they lie in memory, with eight
//     16-byte direct-to-LDS loads, and lane (g, li) reads its column's values
//     back (ds_read2st64 pairs, two k-rows per instruction): 10-17 % faster
//     per block.  The two lane halves read k-rows 4 apart, which share LDS
//     banks; a layout that separated them would give the halves different
//     offsets, and the 2-way conflict costs less than those few reads' issue.
//     At TS = 32 the same route measured no faster (a 16-k deep product's
//     latency is mostly the LDS round trip's).
// Matrix instruction e of unit u then takes k = 8u + e in lanes g = 0 and
// 8u + 4 + e in lanes g = 1, as in gemm32_kernel.  Loads run D - 1 blocks
// ahead of the matrix instructions (a ring of register sets, and for BL of
// LDS stages), either spread over the previous block's matrix instructions
// (IL; one wave per SIMD has no other wave to cover a burst of loads) or
// issued as one burst before them (two waves per SIMD cover each other's
// bursts).  Every block issues the same NL loads, so before a block's B
// values are read from LDS, exactly (D - 2) NL younger loads may still be
// outstanding; the read (read_b_frags) waits for that count itself, since the
// compiler, which tracks which LDS array each direct-to-LDS load writes, loses
// that across the loop's back edge and would wait for every load.
//
// Edges: A's resource ends after row min(M - m0, TS) - 1 at column K, so rows
// past M read zeros; a block's B resource ends at its last k-row below K, so
// k-rows at or past K read zeros, and A's columns at or past K (other data) are
// zeroed before use in the one block that has them.  Columns past N read other
// data but feed only outputs that are not stored.
//
// X3: the same loads feed the 3 x bf16 products instead (gemm32x3_kernel's
// arithmetic).  Per block and 16-k half h, lane (g, li) splits its eight fp32
// values of A's row (units 2h and 2h + 1) and of B's column (the same k) into
// bf16 hi and lo parts; operand slot j < 4 holds k = 16h + 4g + j and slot
// j >= 4 holds k = 16h + 8 + 4g + j - 4, in A and in B alike, so each
// v_mfma_f32_32x32x16_bf16 sums the half's 16 k.  Per 32 x 32 block three
// products, the small terms first (lo.hi, hi.lo, hi.hi).  Half 1's split is
// issued between half 0's matrix instructions.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// One direct-to-LDS 16-byte-per-lane buffer load through the compiler's
// builtin (which, unlike dma16, the compiler counts, so its own load-count
// waits stay exact): lane l's 16 bytes from voffset land at dst + 16 l.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t rsrc, float* dst, int voffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)dst, 16,
                                             voffset, 0, 0, 0);
}

// Lane (g, li)'s B values of one 32 x 64 block from its wave's LDS stage
// (k-row r at r * 64 floats; `base` = the byte address of k-row 4g, column
// li): rb[nj][u][e] = k-row 8u + 4g + e, column 32 nj + li.  One asm
// statement that first waits until at most VM of this wave's vector-memory
// loads are outstanding (so the stage's direct-to-LDS loads have landed) and
// waits for its own reads before it ends, so that no read is in flight when
// the compiler takes the output registers as written.
template <int VM>
__device__ __forceinline__ void read_b_frags64(uint32_t base, uint32_t (&rb)[2][4][4]) {
    // k-row 8u + e is 8u + e rows of 64 floats from base; column block nj
    // 32 floats on.
    u32x2 p[16];
    asm volatile(
        "s_waitcnt vmcnt(%18)\n\t"
        "ds_read2st64_b32 %0, %16 offset0:0 offset1:1\n\t"
        "ds_read2st64_b32 %1, %16 offset0:2 offset1:3\n\t"
        "ds_read2st64_b32 %2, %16 offset0:8 offset1:9\n\t"
        "ds_read2st64_b32 %3, %16 offset0:10 offset1:11\n\t"
        "ds_read2st64_b32 %4, %16 offset0:16 offset1:17\n\t"
        "ds_read2st64_b32 %5, %16 offset0:18 offset1:19\n\t"
        "ds_read2st64_b32 %6, %16 offset0:24 offset1:25\n\t"
        "ds_read2st64_b32 %7, %16 offset0:26 offset1:27\n\t"
        "ds_read2st64_b32 %8, %17 offset0:0 offset1:1\n\t"
        "ds_read2st64_b32 %9, %17 offset0:2 offset1:3\n\t"
        "ds_read2st64_b32 %10, %17 offset0:8 offset1:9\n\t"
        "ds_read2st64_b32 %11, %17 offset0:10 offset1:11\n\t"
        "ds_read2st64_b32 %12, %17 offset0:16 offset1:17\n\t"
        "ds_read2st64_b32 %13, %17 offset0:18 offset1:19\n\t"
        "ds_read2st64_b32 %14, %17 offset0:24 offset1:25\n\t"
        "ds_read2st64_b32 %15, %17 offset0:26 offset1:27\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=v"(p[0]), "=v"(p[1]), "=v"(p[2]), "=v"(p[3]), "=v"(p[4]), "=v"(p[5]), "=v"(p[6]),
          "=v"(p[7]), "=v"(p[8]), "=v"(p[9]), "=v"(p[10]), "=v"(p[11]), "=v"(p[12]),
          "=v"(p[13]), "=v"(p[14]), "=v"(p[15])
        : "v"(base), "v"(base + 128), "n"(VM)
        : "memory");
#pragma unroll
    for (int nj = 0; nj < 2; ++nj)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            rb[nj][u][0] = p[8 * nj + 2 * u][0];
            rb[nj][u][1] = p[8 * nj + 2 * u][1];
            rb[nj][u][2] = p[8 * nj + 2 * u + 1][0];
            rb[nj][u][3] = p[8 * nj + 2 * u + 1][1];
        }
}

template <bool EPI, int MI, int W, bool IL, bool X3>
__global__ __launch_bounds__(64 * W) void gemm32_slicek_kernel(
    const char* __restrict__ A, const char* __restrict__ B, char* __restrict__ C,
    int M, int N, int K, int lda, int ldb, int ldc, int tiles_m, int tiles_n, EpiArgs epi) {
    static_assert((MI == 1 || MI == 2) && (W == 4 || W == 8), "tile and waves");
    constexpr int TS = 32 * MI;
    constexpr int D = MI == 1 ? 3 : 2;  // blocks in the load ring
    constexpr int NB = MI * MI;         // 32 x 32 blocks of the tile
    constexpr bool BL = MI == 2;        // B through LDS
    constexpr int BLK = 32 * TS;        // fp32 of one wave's B block
    constexpr int NLB = BL ? BLK / 256 : MI * 16;  // B loads per block
    __shared__ __attribute__((aligned(1024))) float lb0[BL ? W * BLK : 4];
    __shared__ __attribute__((aligned(1024))) float lb1[BL ? W * BLK : 4];
    __shared__ __attribute__((aligned(1024))) float lb2[BL && D == 3 ? W * BLK : 4];
    __shared__ __attribute__((aligned(16))) float red[W * NB * 16 * 64];
    int tm, tn;
    map_tile((int)blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int lane = (int)threadIdx.x & 63;
    // wave-uniform (so its k range, B's resources and the loop bounds live in
    // scalar registers; taken from threadIdx.x it would count as divergent)
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int g = lane >> 5;
    const int li = lane & 31;
    const int m0 = tm * TS;
    const int n0 = tn * TS;
    const int rows_a = (M - m0) < TS ? (M - m0) : TS;
    const int cols_b = (N - n0) < TS ? (N - n0) : TS;
    const int nblk = (K + 31) / 32;
    const int kb0 = (int)((int64_t)wave * nblk / W);
    const int nb = (int)((int64_t)(wave + 1) * nblk / W) - kb0;
    const int kend = kb0 + nb;

    // BL: global offset (bytes, from the block's corner) that direct-to-LDS
    // load j of this lane fetches: the 4 floats that belong at floats
    // 256 j + 4 lane of the wave's stage.
    int voff_b[BL ? NLB : 1];
#pragma unroll
    for (int j = 0; j < (BL ? NLB : 0); ++j) {
        const int q = 256 * j + 4 * lane;
        voff_b[j] = ((q / TS) * ldb + q % TS) * 4;
    }

    u32x4 ra[D][MI][4];     // [stage][mi][unit]: k 8u + 4g .. + 3 of row mi * 32 + li
    uint32_t rbr[BL ? 1 : D][MI][4][4];  // !BL: [stage][nj][unit][e]: k 8u + 4g + e of column nj * 32 + li
    f32x16 acc[MI][MI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int nj = 0; nj < MI; ++nj)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][nj][r] = 0.0f;

    auto stage = [&](auto set) -> float* {
        constexpr int S = decltype(set)::value;
        return (S == 0 ? lb0 : S == 1 ? lb1 : lb2) + wave * BLK;
    };
    // Block kb's resources.  Blocks past this wave's run get empty ones (their
    // loads return zeros without touching memory), so that every step issues
    // the same loads on every path and the compiler's load-count waits stay
    // exact.
    struct Descs {
        __amdgpu_buffer_rsrc_t a, b;
    };
    auto descs = [&](int kb) {
        const bool live = kb < kend;
        const int k0 = kb * 32;
        const int krows = (K - k0) < 32 ? (K - k0) : 32;
        return Descs{make_rsrc(A + ((int64_t)m0 * lda + k0) * 4,
                               live ? ((int64_t)(rows_a - 1) * lda + krows) * 4 : 0),
                     make_rsrc(B + ((int64_t)k0 * ldb + n0) * 4,
                               live ? ((int64_t)(krows - 1) * ldb + cols_b) * 4 : 0)};
    };
    // Load l of a block into stage S: A's MI * 4 chunks first, then B's NLB.
    constexpr int NL = MI * 4 + NLB;
    constexpr int NM = (X3 ? 6 : 16) * MI * MI;  // matrix instructions per block
    auto load_one = [&](const Descs& d, int l, auto set) {
        constexpr int S = decltype(set)::value;
        if (l < MI * 4) {
            const int u = l / MI, mi = l % MI;
            ra[S][mi][u] = load16(d.a, ((mi * 32 + li) * lda + 8 * u + 4 * g) * 4);
        } else if constexpr (BL) {
            const int j = l - MI * 4;
            lds_load16(d.b, stage(set) + 256 * j, voff_b[j]);
        } else {
            const int q = l - MI * 4;
            const int u = q / (4 * MI), e = (q / MI) % 4, nj = q % MI;
            rbr[S][nj][u][e] = __builtin_amdgcn_raw_buffer_load_b32(
                d.b, ((8 * u + 4 * g + e) * ldb + nj * 32 + li) * 4, 0, 0);
        }
    };
    auto load_block = [&](int kb, auto set) {
        const Descs d = descs(kb);
#pragma unroll
        for (int l = 0; l < NL; ++l) load_one(d, l, set);
    };
    // One block from stage S, with block kb + D - 1's loads (into the stage the
    // previous block emptied) spread over its matrix instructions.
    auto step = [&](int kb, auto set) {
        constexpr int S = decltype(set)::value;
        using SN = std::integral_constant<int, (S + D - 1) % D>;
        const Descs nd = descs(kb + D - 1);
        const int k0 = kb * 32;
        if (k0 + 32 > K) {  // the block holding K's tail: zero A's columns at or past K
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int mi = 0; mi < MI; ++mi)
                    ra[S][mi][u] = mask_tail32(ra[S][mi][u], K - (k0 + 8 * u + 4 * g));
        }
        // B's values of this lane: [nj][unit][e] = k-row 8u + 4g + e, column nj * 32 + li.
        uint32_t rb[MI][4][4];
        if constexpr (BL) {
            read_b_frags64<(D - 2) * NL>(lds_addr((const char*)(stage(set) + 4 * g * TS + li)), rb);
        } else {
#pragma unroll
            for (int nj = 0; nj < MI; ++nj)
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int e = 0; e < 4; ++e) rb[nj][u][e] = rbr[S][nj][u][e];
        }
        if constexpr (!IL) {
#pragma unroll
            for (int l = 0; l < NL; ++l) load_one(nd, l, SN{});
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (X3) {
            // [half][block] hi and lo parts; split c (0 .. 2 MI - 1) of a half
            // is A's block c when c < MI, else B's block c - MI.
            u32x4 hi[2][2][MI], lo[2][2][MI];
            auto split = [&](int h, int c) {
                if (c < MI) {
                    split8(ra[S][c][2 * h], ra[S][c][2 * h + 1], hi[h][0][c], lo[h][0][c]);
                } else {
                    const int nj = c - MI;
                    const u32x4 x = {rb[nj][2 * h][0], rb[nj][2 * h][1], rb[nj][2 * h][2],
                                     rb[nj][2 * h][3]};
                    const u32x4 y = {rb[nj][2 * h + 1][0], rb[nj][2 * h + 1][1],
                                     rb[nj][2 * h + 1][2], rb[nj][2 * h + 1][3]};
                    split8(x, y, hi[h][1][nj], lo[h][1][nj]);
                }
            };
#pragma unroll
            for (int c = 0; c < 2 * MI; ++c) split(0, c);
#pragma unroll
            for (int i = 0; i < NM; ++i) {
                const int h = i / (3 * MI * MI), blk = (i / 3) % (MI * MI), t = i % 3;
                const int mi = blk / MI, nj = blk % MI;
                const u32x4 av = t == 0 ? lo[h][0][mi] : hi[h][0][mi];
                const u32x4 bv = t == 1 ? lo[h][1][nj] : hi[h][1][nj];
                acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv), acc[mi][nj], 0,
                    0, 0);
                __builtin_amdgcn_sched_barrier(0);
                if (h == 0 && i < 2 * MI) split(1, i);
                if constexpr (IL) {
#pragma unroll
                    for (int l = (i * NL) / NM; l < ((i + 1) * NL) / NM; ++l) load_one(nd, l, SN{});
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
            for (int i = 0; i < NM; ++i) {
                const int u = i / (4 * MI * MI), e = (i / (MI * MI)) % 4;
                const int mi = (i / MI) % MI, nj = i % MI;
                acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                    as_float(ra[S][mi][u][e]), as_float(rb[nj][u][e]), acc[mi][nj], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (IL) {
#pragma unroll
                    for (int l = (i * NL) / NM; l < ((i + 1) * NL) / NM; ++l) load_one(nd, l, SN{});
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    load_block(kb0, I0{});
    if constexpr (D == 3) {
        load_block(kb0 + 1, I1{});
        for (int j = 0; j < nb; j += 3) {
            step(kb0 + j, I0{});
            if (j + 1 >= nb) break;
            step(kb0 + j + 1, I1{});
            if (j + 2 >= nb) break;
            step(kb0 + j + 2, I2{});
        }
    } else {
        for (int j = 0; j < nb; j += 2) {
            step(kb0 + j, I0{});
            if (j + 1 >= nb) break;
            step(kb0 + j + 1, I1{});
        }
    }
    // The waves' partial tiles, added in wave order (wave 0's first), each
    // wave summing and storing its share of the tile's accumulator registers:
    // value idx = 16 b + r (block b, register r) of every lane, for idx in
    // [wave PER, wave PER + PER).  Register r of lane (g, li) in block b is
    // row 32 (b / MI) + 8 (r / 4) + 4 g + r % 4, column 32 (b % MI) + li of
    // the tile; stores go through a buffer resource from the tile's corner to
    // the end of C, so rows past M fall outside it, and columns past N get an
    // offset outside any range (the common epilogue's scheme).  BL: the last
    // blocks' direct-to-LDS loads (empty ranges past the run, which still write
    // zeros into the stages) land first, so none is left in flight when the
    // workgroup's LDS is released.
    if constexpr (BL) __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));
    constexpr int PER = NB * 16 / W;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) red[(wave * NB * 16 + b * 16 + r) * 64 + lane] = acc[b / MI][b % MI][r];
    __syncthreads();
    const __amdgpu_buffer_rsrc_t cr = c_rsrc(C, M, N, ldc, m0, n0, 4);
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int idx = wave * PER + q;
        const int b = idx / 16, r = idx % 16;
        float v = red[idx * 64 + lane];
#pragma unroll
        for (int w = 1; w < W; ++w) v += red[(w * NB * 16 + idx) * 64 + lane];
        const int cl = (b % MI) * 32 + li;   // column within the tile
        const uint32_t off =
            (n0 + cl < N ? (uint32_t)((4 * g * ldc + cl) * 4) : OOB_LANE) +
            (uint32_t)(((b / MI) * 32 + 8 * (r >> 2) + (r & 3)) * ldc * 4);
        if constexpr (EPI) {
            const float bias = (epi.bias && n0 + cl < N) ? epi.bias[n0 + cl] : 0.0f;
            v = epilogue_rs<OUT_F32>(v, cr, off, bias, epi);
        }
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), cr, (int)off, 0, 0);
    }
}

hipError_t go(const void* fn, const GemmLaunch& L) {
    const char* a = L.A;
    const char* b = L.B;
    char* c = L.C;
    int M = L.M, N = L.N, K = L.K, lda = L.lda, ldb = L.ldb, ldc = L.ldc;
    int tiles_m = L.tiles_m, tiles_n = L.tiles_n, kchunk = L.kchunk;
    int64_t zs = L.c_zstride;
    EpiArgs e = L.e;
    void* args[] = {&a, &b, &c, &M, &N, &K, &lda, &ldb, &ldc, &tiles_m, &tiles_n, &kchunk, &zs, &e};
    return hipLaunchKernel(fn, dim3((unsigned)(tiles_m * tiles_n), (unsigned)L.splits),
                           dim3(NTHREADS), args, 0, L.stream);
}

// Slice-K launches: one workgroup of W waves per TS x TS tile.
template <int MI, int W, bool IL, bool X3>
hipError_t go_slicek(const GemmLaunch& L) {
    const void* fn = L.epi ? (const void*)gemm32_slicek_kernel<true, MI, W, IL, X3>
                           : (const void*)gemm32_slicek_kernel<false, MI, W, IL, X3>;
    const char* a = L.A;
    const char* b = L.B;
    char* c = L.C;
    int M = L.M, N = L.N, K = L.K, lda = L.lda, ldb = L.ldb, ldc = L.ldc;
    int tiles_m = L.tiles_m, tiles_n = L.tiles_n;
    EpiArgs e = L.e;
    void* args[] = {&a, &b, &c, &M, &N, &K, &lda, &ldb, &ldc, &tiles_m, &tiles_n, &e};
    return hipLaunchKernel(fn, dim3((unsigned)(tiles_m * tiles_n)), dim3(64 * W), args, 0, L.stream);
}

}  // namespace

hipError_t launch_gemm32(const GemmLaunch& L) {
    if (L.out != OUT_F32 || L.tbm != L.tbn) return hipErrorInvalidValue;
    if (L.in == IN_F32 && L.splits == 1 && L.tbm == 32 && L.slice_waves == 4)
        return go_slicek<1, 4, true, false>(L);
    if (L.in == IN_F32 && L.splits == 1 && L.tbm == 32 && L.slice_waves == 8)
        return go_slicek<1, 8, false, false>(L);
    if (L.in == IN_F32 && L.splits == 1 && L.tbm == 64 && L.slice_waves == 4)
        return go_slicek<2, 4, true, false>(L);
    if (L.in == IN_F32X3 && L.splits == 1 && L.tbm == 32 && L.slice_waves == 4)
        return go_slicek<1, 4, true, true>(L);
    if (L.in == IN_F32X3 && L.splits == 1 && L.tbm == 32 && L.slice_waves == 8)
        return go_slicek<1, 8, false, true>(L);
    if (L.in == IN_F32X3 && L.splits == 1 && L.tbm == 64 && L.slice_waves == 4)
        return go_slicek<2, 4, true, true>(L);
    if (L.in == IN_F32 && L.tbm == 128)
        return go(L.epi ? (const void*)gemm32_kernel<true, 128> : (const void*)gemm32_kernel<false, 128>,
                  L);
    if (L.in == IN_F32X3 && L.tbm == 256)
        return go(L.epi ? (const void*)gemm32x3_kernel<true, 256>
                        : (const void*)gemm32x3_kernel<false, 256>, L);
    if (L.in == IN_F32X3 && L.tbm == 128)
        return go(L.epi ? (const void*)gemm32x3_kernel<true, 128>
                        : (const void*)gemm32x3_kernel<false, 128>, L);
    return hipErrorInvalidValue;
}

}  // namespace dgemm
