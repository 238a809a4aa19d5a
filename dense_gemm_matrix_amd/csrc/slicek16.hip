// slicek16.hip -- the bf16 / fp16 slice-K kernel for small outputs on gfx950
// (MI355X).
//
// A product whose output has few 128 x 128 tiles leaves most of the 256 CUs
// idle on the grid kernel; split-K (the nine-levels tutorial, section 2.9)
// fills them only through a caller's workspace and a second kernel.  Here the
// parallelism in K is found inside the workgroup instead, as the fp32
// slice-K kernel in gemm32.hip does: a workgroup of W waves owns a small
// TS x TS tile (TS = 32 MI), each wave takes an equal run of 64-k blocks and
// holds the whole tile's accumulators for its own k, and the W partial tiles
// are added in LDS in wave order, each wave summing and storing (with the
// fused epilogue) an equal share of the tile.  No workspace, no second kernel.
//
// Operands of v_mfma_f32_32x32x16_{bf16,f16}, per 16-k half h of a block:
// lane (g, li) holds k = 16h + 8g .. 16h + 8g + 7 of A's row li and of B's
// column li.  No operand is shared between the waves, so each wave moves its
// own:
//   * A: one 16-byte load per half and 32-row block, straight into the
//     registers the matrix instruction reads (A is K-contiguous).
//   * B is N-contiguous, so a lane's eight k of one column lie in eight rows:
//     the block's 64 k-rows x TS columns go into the wave's own LDS region as
//     they lie in memory (16-byte direct-to-LDS loads, 4 MI per block), and
//     ds_read_b64_tr_b16 transposes on the way back: within each 16-lane
//     group, lane 4a + q addresses k-row a, columns 4q .. 4q + 3 of the
//     group's 16, and lane j receives column j's four consecutive k.  Two such
//     reads give a lane its eight k (the same transpose read as gemm16.hip's).
// Loads run D - 1 blocks ahead (a ring of D register sets for A and D LDS
// stages for B, each stage its own array; D = 3, or 2 for the 64 x 64 tile,
// whose three stages would not fit beside the partial tiles' sum), spread over
// the previous block's matrix instructions (IL, one wave per SIMD) or issued
// as one burst before them (two waves per SIMD).  Every block issues the same
// NL loads, so before a block's B values are read exactly (D - 2) NL younger
// loads may still be outstanding; the read (read_b16) waits for that count
// itself, since the compiler, which tracks which LDS array each direct-to-LDS
// load writes, loses that across the loop's back edge and would wait for
// every load.
//
// Edges: A's resource ends after row min(M - m0, TS) - 1 at column K (rounded
// up to 16 bytes), so rows past M read zeros and A's columns at or past K are
// zeroed in the one block that has them; a block's B resource ends at its last
// k-row below K, so k-rows at or past K read zeros.  Columns past N read other
// data but feed only outputs that are not stored.  Stores go element by
// element through a resource over C, so nothing outside M x N is written.

#include <type_traits>

#include "kern_common.h"

namespace dgemm {
namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Zero the 16-bit elements of an 8-element chunk at and after `valid`
// (valid <= 0: all of them).
__device__ __forceinline__ u32x4 mask_tail16(u32x4 v, int valid) {
    u32x4 out;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t m = (2 * w < valid ? 0x0000ffffu : 0u) | (2 * w + 1 < valid ? 0xffff0000u : 0u);
        out[w] = v[w] & m;
    }
    return out;
}

// One direct-to-LDS 16-byte-per-lane buffer load through the compiler's
// builtin (counted by the compiler, so its own load-count waits stay exact):
// lane l's 16 bytes from voffset land at dst + 16 l.
__device__ __forceinline__ void lds_load16_b(__amdgpu_buffer_rsrc_t rsrc, char* dst, int voffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)dst, 16,
                                             voffset, 0, 0, 0);
}

// Lane (g, li)'s B operands of one 64-k block from its wave's LDS stage
// (k-row r at r * TS elements; `base` = the byte address of this lane's
// transpose-read slot, k-row 8g + a, column 16 (G & 1) + 4q for lane
// 16 G + 4a + q): p[h][t][nj] = k 16h + 8g + 4t .. + 3 of column 32 nj + li.
// One asm statement that first waits until at most VM of this wave's
// vector-memory loads are outstanding (so the stage's direct-to-LDS loads
// have landed) and waits for its own reads before it ends, so that no read is
// in flight when the compiler takes the output registers as written.
template <int MI, int VM>
__device__ __forceinline__ void read_b16(uint32_t base, u32x2 (&p)[4][2][MI]) {
    if constexpr (MI == 1) {
        // byte offset of (h, t): (16h + 4t) rows of 64 bytes
        asm volatile(
            "s_waitcnt vmcnt(%9)\n\t"
            "ds_read_b64_tr_b16 %0, %8 offset:0\n\t"
            "ds_read_b64_tr_b16 %1, %8 offset:256\n\t"
            "ds_read_b64_tr_b16 %2, %8 offset:1024\n\t"
            "ds_read_b64_tr_b16 %3, %8 offset:1280\n\t"
            "ds_read_b64_tr_b16 %4, %8 offset:2048\n\t"
            "ds_read_b64_tr_b16 %5, %8 offset:2304\n\t"
            "ds_read_b64_tr_b16 %6, %8 offset:3072\n\t"
            "ds_read_b64_tr_b16 %7, %8 offset:3328\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=v"(p[0][0][0]), "=v"(p[0][1][0]), "=v"(p[1][0][0]), "=v"(p[1][1][0]),
              "=v"(p[2][0][0]), "=v"(p[2][1][0]), "=v"(p[3][0][0]), "=v"(p[3][1][0])
            : "v"(base), "n"(VM)
            : "memory");
    } else {
        // byte offset of (h, t, nj): (16h + 4t) rows of 128 bytes, + 64 nj
        asm volatile(
            "s_waitcnt vmcnt(%17)\n\t"
            "ds_read_b64_tr_b16 %0, %16 offset:0\n\t"
            "ds_read_b64_tr_b16 %1, %16 offset:64\n\t"
            "ds_read_b64_tr_b16 %2, %16 offset:512\n\t"
            "ds_read_b64_tr_b16 %3, %16 offset:576\n\t"
            "ds_read_b64_tr_b16 %4, %16 offset:2048\n\t"
            "ds_read_b64_tr_b16 %5, %16 offset:2112\n\t"
            "ds_read_b64_tr_b16 %6, %16 offset:2560\n\t"
            "ds_read_b64_tr_b16 %7, %16 offset:2624\n\t"
            "ds_read_b64_tr_b16 %8, %16 offset:4096\n\t"
            "ds_read_b64_tr_b16 %9, %16 offset:4160\n\t"
            "ds_read_b64_tr_b16 %10, %16 offset:4608\n\t"
            "ds_read_b64_tr_b16 %11, %16 offset:4672\n\t"
            "ds_read_b64_tr_b16 %12, %16 offset:6144\n\t"
            "ds_read_b64_tr_b16 %13, %16 offset:6208\n\t"
            "ds_read_b64_tr_b16 %14, %16 offset:6656\n\t"
            "ds_read_b64_tr_b16 %15, %16 offset:6720\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=v"(p[0][0][0]), "=v"(p[0][0][1]), "=v"(p[0][1][0]), "=v"(p[0][1][1]),
              "=v"(p[1][0][0]), "=v"(p[1][0][1]), "=v"(p[1][1][0]), "=v"(p[1][1][1]),
              "=v"(p[2][0][0]), "=v"(p[2][0][1]), "=v"(p[2][1][0]), "=v"(p[2][1][1]),
              "=v"(p[3][0][0]), "=v"(p[3][0][1]), "=v"(p[3][1][0]), "=v"(p[3][1][1])
            : "v"(base), "n"(VM)
            : "memory");
    }
}

template <int IN>
__device__ __forceinline__ f32x16 mfma16(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (IN == IN_BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <int IN, int OUT, bool EPI, int MI, int W, bool IL>
__global__ __launch_bounds__(64 * W) void slicek16_kernel(
    const char* __restrict__ A, const char* __restrict__ B, char* __restrict__ C,
    int M, int N, int K, int lda, int ldb, int ldc, int tiles_m, int tiles_n, EpiArgs epi) {
    static_assert((MI == 1 || MI == 2) && (W == 4 || W == 8), "tile and waves");
    constexpr int TS = 32 * MI;
    constexpr int D = MI == 1 ? 3 : 2;   // blocks in the load ring
    constexpr int NB = MI * MI;          // 32 x 32 blocks of the tile
    constexpr int BLKB = 128 * TS;       // bytes of one wave's B block: 64 k-rows x TS
    constexpr int NDB = BLKB / 1024;     // its direct-to-LDS loads
    constexpr int NL = 4 * MI + NDB;     // loads per block: A's 4 MI chunks, then B's
    constexpr int NM = 4 * NB;           // matrix instructions per block
    constexpr int ES = OUT == OUT_F32 ? 4 : 2;
    __shared__ __attribute__((aligned(1024))) char lb0[W * BLKB];
    __shared__ __attribute__((aligned(1024))) char lb1[W * BLKB];
    __shared__ __attribute__((aligned(1024))) char lb2[D == 3 ? W * BLKB : 16];
    __shared__ __attribute__((aligned(16))) float red[W * NB * 16 * 64];
    int tm, tn;
    map_tile((int)blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int lane = (int)threadIdx.x & 63;
    // wave-uniform (so its k range, the resources and the loop bounds live in
    // scalar registers; taken from threadIdx.x it would count as divergent)
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int g = lane >> 5;
    const int li = lane & 31;
    const int m0 = tm * TS;
    const int n0 = tn * TS;
    const int rows_a = (M - m0) < TS ? (M - m0) : TS;
    const int cols_b = (N - n0) < TS ? (N - n0) : TS;
    const int nblk = (K + 63) / 64;
    const int kb0 = (int)((int64_t)wave * nblk / W);
    const int nb = (int)((int64_t)(wave + 1) * nblk / W) - kb0;
    const int kend = kb0 + nb;

    // Global offset (bytes, from the block's corner) that direct-to-LDS load j
    // of this lane fetches: the 16 bytes that belong at bytes 1024 j + 16 lane
    // of the wave's stage (k-row q / 2TS, byte q % 2TS of the row).
    int voff_b[NDB];
#pragma unroll
    for (int j = 0; j < NDB; ++j) {
        const int q = 1024 * j + 16 * lane;
        voff_b[j] = (q / (2 * TS)) * ldb * 2 + q % (2 * TS);
    }
    // This lane's transpose-read slot: lane 16 G + 4a + q reads k-row 8 (G / 2) + a,
    // columns 16 (G & 1) + 4q .. + 3.
    const int grp = lane >> 4;
    const uint32_t rd_slot =
        (uint32_t)(((8 * (grp >> 1) + ((lane >> 2) & 3)) * TS + 16 * (grp & 1) + 4 * (lane & 3)) * 2);

    u32x4 ra[D][MI][4];  // [stage][mi][h]: k 16h + 8g .. + 7 of row mi * 32 + li
    f32x16 acc[MI][MI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int nj = 0; nj < MI; ++nj)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][nj][r] = 0.0f;

    auto stage = [&](auto set) -> char* {
        constexpr int S = decltype(set)::value;
        return (S == 0 ? lb0 : S == 1 ? lb1 : lb2) + wave * BLKB;
    };
    // Block kb's resources.  Blocks past this wave's run get empty ones (their
    // loads return zeros without touching memory), so that every step issues
    // the same loads on every path.
    struct Descs {
        __amdgpu_buffer_rsrc_t a, b;
    };
    auto descs = [&](int kb) {
        const bool live = kb < kend;
        const int k0 = kb * 64;
        const int krows = (K - k0) < 64 ? (K - k0) : 64;
        return Descs{make_rsrc(A + ((int64_t)m0 * lda + k0) * 2,
                               live ? ((int64_t)(rows_a - 1) * lda + krows) * 2 : 0),
                     make_rsrc(B + ((int64_t)k0 * ldb + n0) * 2,
                               live ? ((int64_t)(krows - 1) * ldb + cols_b) * 2 : 0)};
    };
    auto load_one = [&](const Descs& d, int l, auto set) {
        constexpr int S = decltype(set)::value;
        if (l < 4 * MI) {
            const int h = l / MI, mi = l % MI;
            ra[S][mi][h] = load16(d.a, ((mi * 32 + li) * lda + 16 * h + 8 * g) * 2);
        } else {
            const int j = l - 4 * MI;
            lds_load16_b(d.b, stage(set) + 1024 * j, voff_b[j]);
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
        const int k0 = kb * 64;
        if (k0 + 64 > K) {  // the block holding K's tail: zero A's columns at or past K
#pragma unroll
            for (int h = 0; h < 4; ++h)
#pragma unroll
                for (int mi = 0; mi < MI; ++mi)
                    ra[S][mi][h] = mask_tail16(ra[S][mi][h], K - (k0 + 16 * h + 8 * g));
        }
        u32x2 p[4][2][MI];
        read_b16<MI, (D - 2) * NL>(lds_addr(stage(set)) + rd_slot, p);
        if constexpr (!IL) {
#pragma unroll
            for (int l = 0; l < NL; ++l) load_one(nd, l, SN{});
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            const int h = i / NB, mi = (i / MI) % MI, nj = i % MI;
            const u32x4 b = {p[h][0][nj][0], p[h][0][nj][1], p[h][1][nj][0], p[h][1][nj][1]};
            acc[mi][nj] = mfma16<IN>(ra[S][mi][h], b, acc[mi][nj]);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (IL) {
#pragma unroll
                for (int l = (i * NL) / NM; l < ((i + 1) * NL) / NM; ++l) load_one(nd, l, SN{});
            }
            __builtin_amdgcn_sched_barrier(0);
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
    // offset outside any range (the common epilogue's scheme).
    // The last blocks' direct-to-LDS loads (empty ranges past the run, which
    // still write zeros into the stages) land before the wave goes on, so none
    // is left in flight when the workgroup's LDS is released.
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));
    constexpr int PER = NB * 16 / W;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            red[(wave * NB * 16 + b * 16 + r) * 64 + lane] = acc[b / MI][b % MI][r];
    __syncthreads();
    const __amdgpu_buffer_rsrc_t cr = c_rsrc(C, M, N, ldc, m0, n0, ES);
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int idx = wave * PER + q;
        const int b = idx / 16, r = idx % 16;
        float v = red[idx * 64 + lane];
#pragma unroll
        for (int w = 1; w < W; ++w) v += red[(w * NB * 16 + idx) * 64 + lane];
        const int cl = (b % MI) * 32 + li;  // column within the tile
        const uint32_t off =
            (n0 + cl < N ? (uint32_t)((4 * g * ldc + cl) * ES) : OOB_LANE) +
            (uint32_t)(((b / MI) * 32 + 8 * (r >> 2) + (r & 3)) * ldc * ES);
        if constexpr (EPI) {
            const float bias = (epi.bias && n0 + cl < N) ? epi.bias[n0 + cl] : 0.0f;
            v = epilogue_rs<OUT>(v, cr, off, bias, epi);
        }
        if constexpr (OUT == OUT_F32)
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), cr, (int)off, 0, 0);
        else
            __builtin_amdgcn_raw_buffer_store_b16((unsigned short)pack16<OUT>(v, 0.0f), cr, (int)off,
                                                  0, 0);
    }
}

template <int IN, int OUT, int MI, int W, bool IL>
hipError_t go_slice16(const GemmLaunch& L) {
    const void* fn = L.epi ? (const void*)slicek16_kernel<IN, OUT, true, MI, W, IL>
                           : (const void*)slicek16_kernel<IN, OUT, false, MI, W, IL>;
    const char* a = L.A;
    const char* b = L.B;
    char* c = L.C;
    int M = L.M, N = L.N, K = L.K, lda = L.lda, ldb = L.ldb, ldc = L.ldc;
    int tiles_m = L.tiles_m, tiles_n = L.tiles_n;
    EpiArgs e = L.e;
    void* args[] = {&a, &b, &c, &M, &N, &K, &lda, &ldb, &ldc, &tiles_m, &tiles_n, &e};
    return hipLaunchKernel(fn, dim3((unsigned)(tiles_m * tiles_n)), dim3(64 * W), args, 0, L.stream);
}

template <int IN, int OUT>
hipError_t slice16_by_variant(const GemmLaunch& L) {
    if (L.tbm == 32 && L.slice_waves == 4) return go_slice16<IN, OUT, 1, 4, true>(L);
    if (L.tbm == 32 && L.slice_waves == 8) return go_slice16<IN, OUT, 1, 8, false>(L);
    if (L.tbm == 64 && L.slice_waves == 4) return go_slice16<IN, OUT, 2, 4, true>(L);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_slicek16(const GemmLaunch& L) {
    if (L.splits != 1 || L.tbm != L.tbn) return hipErrorInvalidValue;
    if (L.in == IN_BF16 && L.out == OUT_F32) return slice16_by_variant<IN_BF16, OUT_F32>(L);
    if (L.in == IN_BF16 && L.out == OUT_BF16) return slice16_by_variant<IN_BF16, OUT_BF16>(L);
    if (L.in == IN_F16 && L.out == OUT_F32) return slice16_by_variant<IN_F16, OUT_F32>(L);
    if (L.in == IN_F16 && L.out == OUT_F16) return slice16_by_variant<IN_F16, OUT_F16>(L);
    return hipErrorInvalidValue;
}

}  // namespace dgemm
