// dgemm_internal.h -- what the library's translation units share: format
// codes, the workgroup -> tile map, the epilogue arguments, and one launch
// description per kernel family.  Host-visible; no device code.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace dgemm {

enum InFmt { IN_F32 = 0, IN_BF16 = 1, IN_F16 = 2, IN_F32X3 = 3 };  // F32X3: fp32 via 3 x bf16
enum OutFmt { OUT_F32 = 0, OUT_BF16 = 1, OUT_F16 = 2 };

constexpr int NTHREADS = 256;   // 4 waves: the fp32 kernels' workgroup
constexpr int GROUP_M = 4;      // tile rows per strip in the tile walk
constexpr int NUM_XCD = 8;      // XCDs that workgroups are dealt across
constexpr int NUM_CU = 256;     // compute units of an MI355X

inline int in_esize(int in) { return (in == IN_F32 || in == IN_F32X3) ? 4 : 2; }
inline int out_esize(int out) { return out == OUT_F32 ? 4 : 2; }

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

// Fused epilogue: C := act(alpha * acc + beta * C_old + bias[col]).  C_old is
// read only when beta != 0; bias may be NULL; relu != 0 clamps negatives to 0.
struct EpiArgs {
    float alpha;
    float beta;
    const float* bias;
    int relu;
};

// One GEMM launch.  The grid is (tiles_m * tiles_n, splits): workgroup
// (x, z) computes tile map_tile(x) over k in [z * kchunk, min(K, (z + 1) *
// kchunk)) and writes it at C + z * c_zstride bytes.  Unsplit launches have
// splits = 1 and kchunk = K.
struct GemmLaunch {
    int in, out, tbm, tbn;
    int stages;  // LDS stages of the 16-bit kernel's 128 x 128 tile (2, or 4 alone on a CU)
    int slice_waves;  // waves per workgroup of a slice-K launch (0: a grid launch)
    bool epi;    // apply `e` in the kernel (only with splits == 1)
    const char* A;
    const char* B;
    char* C;
    int M, N, K, lda, ldb, ldc;
    int tiles_m, tiles_n, splits, kchunk;
    int64_t c_zstride;
    EpiArgs e;
    hipStream_t stream;
};

// ------------------------------------------------------------------ Stream-K
//
// The nine-levels tutorial's section 2.9 names Stream-K as the refinement of
// Split-K that gives every thread block the same amount of work.  Here, for
// grids of at most one 256 x 256 tile per CU (the 16-bit kernel's tile), a
// persistent grid of G workgroups (G a multiple of the 8 XCDs, one per CU):
// the tiles map_tile gives XCD x (tile walk positions x + 8 u, u < n_x) are
// laid end to end as W = n_x nk iterations (one iteration = one 64-k step of
// one tile), and XCD x's R = G / 8 workgroups (b = x + 8 j, rank j) take
// consecutive runs of equal length: rank j covers [floor(j W / R),
// floor((j + 1) W / R)).  The host keeps n_x <= R (so a run is at most nk
// iterations long and touches at most two tiles) and W >= R (so no run is
// empty).
//
// A rank computes the pieces of its run (one or two: the k range it holds of
// each tile it touches) into fp32 partial-tile slots, then publishes them with
// one flag.  Each tile is then reduced by all of its contributors together:
// the tile's 64 blocks of 32 x 32 outputs are dealt out in equal runs, and the
// i-th of its n contributors sums its blocks' partials in contributor order
// (k order), applies the epilogue and stores them.  Every output is so added
// in one fixed order whatever the timing: a deterministic fix-up with no
// atomic arithmetic, whose reads are shared evenly by the workgroups of the
// tile.  All contributors of a tile are on one XCD, so partial sums meet in
// that XCD's L2.
//
// Waits are bounded: a reducer waits for a contributor's flag at most
// wait_ticks (wall-clock ticks); a piece that has not appeared by then (its
// rank has not started, for instance because the grid is not co-resident) the
// reducer computes itself, into that rank's slot, with the same code on the
// same data: the bits the contributor writes, so a late contributor
// overwrites them with themselves.  No wait can therefore hang the kernel, and
// the output never depends on which path ran.  A flag holds the launch's
// 64-bit epoch (a new value per launch from the host), so flags left by
// earlier launches in the workspace are never taken for this launch's.
//
// part: 2 G fp32 tiles of 256 KiB (slots 2 b and 2 b + 1: workgroup b's first
// and second piece); flags: G 64-bit words.
struct SkSched {
    int tiles_m, tiles_n;
    int nk;         // 64-k steps per tile
    char* part;
    unsigned long long* flags;
    unsigned long long epoch;
    long long wait_ticks;
};

constexpr int SK_TILE = 256;    // the Stream-K macro-tile, square
constexpr int SK_BK = 64;       // k per iteration
constexpr int SK_BLOCKS = 64;   // 32 x 32 output blocks per tile

// Rank j of XCD x and its run [s0, s1) of the XCD's W iterations.
struct SkRun {
    int x, j, R, nk, W, s0, s1;
    int u0;        // the tile of the first piece (of the XCD's list)
    int npieces;   // 1 or 2 (the second: tile u0 + 1)
    __host__ __device__ int start(int r) const { return (int)((int64_t)r * W / R); }
    __host__ __device__ int pos(int u) const { return x + NUM_XCD * u; }  // tile walk position
    __host__ __device__ int rank_of(int it) const {  // the rank whose run holds iteration it
        return (int)((((int64_t)it + 1) * R - 1) / W);
    }
    __host__ __device__ int first(int u) const { return rank_of(u * nk); }
    __host__ __device__ int last(int u) const { return rank_of((u + 1) * nk - 1); }
    // Slot of rank p's piece of tile u.
    __host__ __device__ int slot(int p, int u) const {
        return 2 * (x + NUM_XCD * p) + (start(p) / nk == u ? 0 : 1);
    }
    // Rank p's k range [kb, ke) of tile u, in iterations of the tile.
    __host__ __device__ void piece(int p, int u, int& kb, int& ke) const {
        const int t0 = u * nk;
        const int a = start(p), b = start(p + 1);
        kb = (a > t0 ? a : t0) - t0;
        ke = (b < t0 + nk ? b : t0 + nk) - t0;
    }
};

__host__ __device__ inline SkRun sk_run(const SkSched& sk, int b, int G) {
    SkRun r;
    r.x = b % NUM_XCD;
    r.j = b / NUM_XCD;
    r.R = G / NUM_XCD;
    r.nk = sk.nk;
    const int tiles = sk.tiles_m * sk.tiles_n;
    const int nx = tiles > r.x ? (tiles - r.x + NUM_XCD - 1) / NUM_XCD : 0;
    r.W = nx * sk.nk;
    r.s0 = r.start(r.j);
    r.s1 = r.start(r.j + 1);
    r.u0 = r.W > 0 ? r.s0 / sk.nk : 0;
    r.npieces = r.W == 0 ? 0 : (r.s1 > (r.u0 + 1) * sk.nk ? 2 : 1);
    return r;
}

// Blocks [lo, hi) of tile u that rank j reduces: its share among the tile's
// contributors first(u) .. last(u).
__host__ __device__ inline void sk_share(const SkRun& r, int u, int& lo, int& hi) {
    const int f = r.first(u), n = r.last(u) - f + 1, i = r.j - f;
    lo = SK_BLOCKS * i / n;
    hi = SK_BLOCKS * (i + 1) / n;
}

// Workspace of a Stream-K launch of `grid` workgroups: 2 grid partial tiles,
// then one 64-bit flag per workgroup.
constexpr int64_t sk_ws_bytes(int grid) {
    return (int64_t)2 * grid * SK_TILE * SK_TILE * 4 + (int64_t)grid * 8;
}

// Per kernel family; each returns hipErrorInvalidValue for a combination it
// has no instantiation for.
hipError_t launch_gemm16(const GemmLaunch& L);  // IN_BF16, IN_F16
// The Stream-K launch: L as for launch_gemm16 with tbm = tbn = 256 and
// splits = 1; `grid` workgroups, a multiple of NUM_XCD.
hipError_t launch_gemm16_sk(const GemmLaunch& L, const SkSched& s, int grid);
hipError_t launch_gemm32(const GemmLaunch& L);  // IN_F32, IN_F32X3
hipError_t launch_slicek16(const GemmLaunch& L);  // IN_BF16, IN_F16 with slice_waves > 0

// Split-K reduction: C[i][j] = epilogue(sum_{z < splits} W[z][i][j]) with W
// fp32, row pitch ldw (a multiple of 4) and split stride zstride elements.
hipError_t launch_splitk_reduce(const float* W, int splits, int64_t zstride, int ldw, char* C,
                                int ldc, int M, int N, int out, bool epi, const EpiArgs& e,
                                hipStream_t stream);

}  // namespace dgemm
