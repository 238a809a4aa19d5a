// dgemm.hip -- the C ABI of include/dgemm.h: argument validation, the launch
// plan (macro-tile shape and split-K count) and the kernel launches.  Host
// code only; the kernels live in gemm16.hip (bf16 / fp16), gemm32.hip (fp32,
// and fp32 via 3 x bf16) and splitk.hip (the split-K reduction).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "dgemm.h"
#include "dgemm_internal.h"

namespace dgemm {
namespace {

constexpr int64_t DESC_LIMIT = (int64_t)1 << 31;  // 32-bit buffer offsets
constexpr int PANEL_ROWS = 256;                   // rows of A one descriptor spans

// K per step: the k rows of B one descriptor spans.
int bk_of(int in) { return (in == IN_BF16 || in == IN_F16) ? 64 : 32; }

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

// The bytes a row-major operand occupies: `rows` rows of `row_bytes` each,
// `pitch` bytes apart.  A contiguous range is one row.
struct Span {
    uintptr_t base;
    int64_t rows, row_bytes, pitch;
};

Span matrix_span(const void* p, int64_t rows, int64_t cols, int64_t ld, int64_t esize) {
    return Span{(uintptr_t)p, rows, cols * esize, ld * esize};
}

int64_t floor_div(int64_t a, int64_t b) {  // b > 0
    return a >= 0 ? a / b : -((-a + b - 1) / b);
}

// Whether any byte of x's rows is also a byte of y's rows.  With equal pitches
// (a one-row span takes the other's pitch) row i of x and row j of y overlap
// iff -x.row_bytes < (x.base - y.base) + (i - j) * pitch < y.row_bytes, which is
// decided for the t = i - j closest to the upper bound.  With different pitches
// the two spans are compared from their first to their last byte, which may
// report an overlap of interleaved rows that share no byte.
bool spans_overlap(Span x, Span y) {
    if (x.rows <= 0 || y.rows <= 0 || x.row_bytes <= 0 || y.row_bytes <= 0) return false;
    const int64_t xlen = (x.rows - 1) * x.pitch + x.row_bytes;
    const int64_t ylen = (y.rows - 1) * y.pitch + y.row_bytes;
    if (!ranges_overlap(x.base, xlen, y.base, ylen)) return false;
    if (x.rows == 1) x.pitch = y.pitch;
    if (y.rows == 1) y.pitch = x.pitch;
    if (x.pitch != y.pitch || x.pitch <= 0) return true;
    const int64_t p = x.pitch;
    const int64_t d = (int64_t)(x.base - y.base);
    const int64_t t = std::min(floor_div(y.row_bytes - 1 - d, p), x.rows - 1);
    if (t < -(y.rows - 1)) return false;
    return d + t * p > -x.row_bytes;
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
        const Span c = matrix_span(C, M, N, ldc, es_out);
        if (spans_overlap(c, matrix_span(A, M, K, lda, es)) ||
            spans_overlap(c, matrix_span(B, K, N, ldb, es)))
            return DGEMM_ERR_ALIAS;
    }
    // Buffer descriptors address one 256-row panel of A, one K step of B (64
    // rows of 16-bit data, 32 of fp32) and one 256-row panel of C with 32-bit
    // offsets.
    if ((int64_t)PANEL_ROWS * lda * es >= DESC_LIMIT || (int64_t)bk_of(in) * ldb * es >= DESC_LIMIT ||
        (int64_t)PANEL_ROWS * ldc * es_out >= DESC_LIMIT)
        return DGEMM_ERR_TOO_LARGE;
    return DGEMM_OK;
}

// ------------------------------------------------------------------ planning
//
// Macro-tile and split-K choice by an estimated time: for a candidate tile
// (with a measured relative per-tile efficiency) and split count s,
//
//   rounds * (steps_per_split * step_us * area / 256^2 / eff + WG_FIXED_US)
//     + (s > 1 ? REDUCE_FIXED_US + reduce_bytes / HBM_BYTES_PER_US : 0)
//
// where step_us is the measured time of one K step of a 256 x 256 workgroup,
// eff the tile's measured throughput relative to it (one workgroup per CU),
// reduce_bytes counts the partial sums written and read back plus C, and
// rounds = ceil(tiles * s / 256) workgroups per CU.  A grid of at most one
// workgroup per CU uses `eff1` in place of eff: the 16-bit 128 x 128 tile then
// runs with a deeper LDS ring (4 stages), which only fits one workgroup per CU,
// and the 3 x bf16 one is measured faster alone on its CU than its pair factor
// implies.
//
// 128 x 128 tiles fit two workgroups on a CU: two co-resident ones take `pair`
// times as long as one alone (bf16 1.26, fp32 1.5, 3 x bf16 1.22), so for them
// rounds counts pairs and the term in parentheses is multiplied by `pair`.
// Grids of two or more rounds of pairs use `pair2`: for 16-bit inputs 1.35 (a
// full round of pairs measured 1.32-1.37 on the multi-round shapes below); for
// the other formats the same as `pair`, their sweeps not separating the two.
//
// Partly filled last rounds (16-bit 256 x 256 and 192 x 256 tiles): a last
// round that fills a fraction f of the CUs counts `last + (1 - last) * f` of a
// full round, last = 0.6.  Under the power cap a partly filled chip runs at a
// higher clock, so a grid of 1.25 rounds takes ~1.7 times one round, not 2.
// The rule prices the unsplit tile choice (`pick_tile`) only; the split-K
// choice keeps whole rounds, as in the sweeps it was fitted to (with the rule
// there, two K = 16384 shapes dropped a 2-way split that is 4-6 % faster).
// Measured on 36 unsplit bf16 shapes from 2048 x 8192 to 8192^2 at K = 2048
// and 4096: with `pair2` and this rule the planner picks the fastest of the
// three tiles on every one (before them, 14 chose 128 x 128 tiles 6-11 %
// slower than the best); on 15 more shapes whose tile they change, the new
// tile is 1-20 % faster.  The 3 x bf16 256 x 256 tile keeps whole rounds: its
// second round costs ~0.6 of the first whatever its fill, but on the shapes
// where a partial-round rule would pick it, its 128 x 128 tile is as fast.
//
// A grid of fewer tiles than CUs, or K much deeper than M and N, is where
// splitting pays (the nine-levels tutorial's section 2.9 names Split-K for
// small-matrix parallelism); everywhere else the unsplit plan wins.  The
// constants were fitted to sweeps of forced plans (every candidate tile, split
// counts 1 to 16, each timed twice).  The latest, 23 bf16 shapes from 512^3 to
// 16384 x 4096 x 4096: the chosen plan is the fastest one timed on 20 of the 22
// shapes whose plan was among those timed and within 2.4 % on the other two;
// fp32 (9 shapes): the fastest on all; 3 x bf16 (12 shapes, after the 128 x 128
// tile's two staging sets): the fastest on 10, within 7.2 % on all.

constexpr int MAX_SPLITS = 16;
constexpr double WG_FIXED_US = 1.0;       // prologue + epilogue per round of workgroups
constexpr double REDUCE_FIXED_US = 3.0;   // launch and tail of the reduction kernel
constexpr double HBM_BYTES_PER_US = 5.0e6;
constexpr double SPLIT_MARGIN = 0.9;      // a split plan must be predicted 10% faster

// pair = 0: one workgroup per CU.  fp32 has the 128 x 128 tile only: in a
// sweep of forced plans 256 x 256 was slower at every shape (4096^3: 1049 us
// against 1002 us), and the cost model never chose it; eff stays relative to
// a 256 x 256 workgroup so that step_us keeps one meaning.
// `pair2`: the pair factor of grids of two or more rounds of pairs; `last`: the
// cost of a last, partly filled round at zero fill (1: whole rounds).
struct TileCand { int bm, bn; double eff, pair, pair2, eff1, last; };
constexpr TileCand TILES16[] = {{256, 256, 1.0, 0.0, 0.0, 1.0, 0.6},
                                {192, 256, 0.95, 0.0, 0.0, 0.95, 0.6},
                                {128, 128, 0.6, 1.26, 1.35, 0.8, 1.0}};
constexpr TileCand TILES32[] = {{128, 128, 0.85, 1.5, 1.5, 0.85, 1.0}};
constexpr TileCand TILES32X3[] = {{256, 256, 1.0, 0.0, 0.0, 1.0, 1.0},
                                  {128, 128, 0.5, 1.22, 1.22, 0.6, 1.0}};

// Workgroup rounds per CU for `wgs` workgroups, and the time factor of a round;
// `partial`: price a partly filled last round by the tile's `last`.
double rounds_factor(const TileCand& t, int64_t wgs, bool partial = false) {
    const int64_t per_cu = (wgs + NUM_CU - 1) / NUM_CU;
    if (t.pair > 0.0 && per_cu >= 2) {
        const int64_t pairs = (per_cu + 1) / 2;
        return (double)pairs * (pairs >= 2 ? t.pair2 : t.pair);
    }
    if (partial && per_cu >= 2 && t.last < 1.0) {
        const double fill = (double)(wgs - (per_cu - 1) * NUM_CU) / NUM_CU;
        return (double)(per_cu - 1) + t.last + (1.0 - t.last) * fill;
    }
    return (double)per_cu;
}

// Throughput of tile t relative to a 256 x 256 workgroup in a grid of `wgs`.
double tile_eff(const TileCand& t, int64_t wgs) { return wgs <= NUM_CU ? t.eff1 : t.eff; }

// Candidate macro-tiles of an input format's kernel.
const TileCand* tiles_for(int in, int& n) {
    if (in == IN_BF16 || in == IN_F16) { n = 3; return TILES16; }
    if (in == IN_F32) { n = 1; return TILES32; }
    n = 2;
    return TILES32X3;
}

// Microseconds per K step of one 256 x 256 workgroup at 4096^3.
double step_us(int in) {
    switch (in) {
    case IN_BF16:
    case IN_F16: return 1.7;   // BK 64
    case IN_F32X3: return 3.5; // BK 32, three bf16 products per term
    default: return 8.3;       // BK 32, fp32 matrix instruction
    }
}

enum PlanKind { PLAN_GRID = 0, PLAN_STREAM_K = 1 };

struct Plan {
    int bm, bn;
    int splits, kchunk;   // kchunk: K per split (a multiple of the K step)
    int ldw;              // row pitch of the fp32 partials, in elements
    int64_t ws_bytes;     // workspace the plan uses (0 when unsplit)
    int kind = PLAN_GRID;
    int waves = 0;        // slice-K plans: waves per workgroup (0: a grid plan)
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ------------------------------------------------------------------ slice-K
//
// fp32 and 3 x bf16 products whose 128 x 128 grid would leave most CUs idle
// (512^3 has 16 such tiles for 256 CUs) run the slice-K kernel instead: 32 x 32
// or 64 x 64 tiles, K split over the W waves of each workgroup and summed in
// LDS, so the grid fills the chip without a workspace or a reduction kernel.
// Estimated time, per input format and candidate, fitted to a sweep of 22
// shapes from 128^3 to 2048^2 x 1024 (MI355X; every candidate plan timed by
// graph replay; worst error 4.5-14 %):
//
//   fixed_us + nbw * blk_us * load + (n - 1) * round_us
//
// with nbw = the 32-k blocks of one wave (ceil(ceil(K / 32) / W)), n =
// ceil(tiles / 256) workgroups per CU, and load = 1 for n = 1, else n * co:
// co < 1 where several workgroups fit on a CU at once (the 4-wave 32 x 32
// kernel) and overlap.  The 32 x 32 tile takes 4 waves (loads spread over the
// matrix instructions) or 8 (two waves per SIMD; faster once K is deep),
// whichever is estimated faster; the 64 x 64 tile takes 4.  The tile itself
// depends on M and N only (the smaller per-block cost of 4 waves), so that
// dgemm_tile_map stays exact.  Against the grid plans the estimate is compared
// like any other: in the sweep slice-K was 1.3-5x faster than the best grid
// plan on small outputs and deep-K shapes without a workspace (3 x bf16 512^3
// 5.2 against 13.1 us, 512 x 512 x 4096 23 against 109 us unsplit), and split-K
// kept the deepest shapes when a workspace is offered (256 x 256 x 8192 3 x bf16
// 25.5 against 40 us).

// fill_us: the per-block cost added at a full round, in proportion to the
// fraction of the CUs the grid fills (0: none measured).
struct SliceCand { int ts, waves; double fixed_us, blk_us, co, round_us, fill_us; };
// fp32 matrix instruction: 32 x 32 with 4 or 8 waves, 64 x 64 with 4.
constexpr SliceCand SLICE_F32[] = {{32, 4, 2.4, 0.9, 0.82, 0.1, 0.0},
                                   {32, 8, 2.7, 1.35, 1.0, 1.6, 0.0},
                                   {64, 4, 3.7, 2.27, 1.0, 4.6, 0.0}};
// 3 x bf16: the same tiles.
constexpr SliceCand SLICE_X3[] = {{32, 4, 2.4, 0.72, 0.86, 0.1, 0.0},
                                  {32, 8, 2.5, 1.19, 1.0, 1.6, 0.0},
                                  {64, 4, 3.6, 1.28, 1.04, 2.9, 0.0}};
// bf16 / fp16 (blocks of 64 k): the same tiles; 8 waves were never faster
// than 4 in the sweep (the 64 x 64 tile's rounds are not fitted: at most 64
// tiles of 128 x 128 give it one round).  The 64 x 64 tile's cost per block
// rises with the grid's fill: 1.08-1.18 us at 64-128 workgroups, 1.14-1.16 at
// 192, 1.18-1.27 at 256 (a full chip clocks lower), so 1.08 + 0.15 * fill.
// With the flat 1.14 it kept 1024 x 1024 x 4096, 512 x 2048 x 4096 and
// 256 x 4096 x 4096 on slice-K (23.3 us) when 4 splits of 128 x 128 tiles
// take 19.8.
constexpr SliceCand SLICE_16[] = {{32, 4, 2.45, 0.60, 1.04, 0.6, 0.0},
                                  {32, 8, 2.45, 1.22, 1.08, 1.4, 0.0},
                                  {64, 4, 3.0, 1.08, 1.0, 2.9, 0.15}};

bool slice_format(int in) { (void)in; return true; }

// K per slice-K block: 64 for 16-bit inputs, 32 for fp32 data.
int slice_bk(int in) { return (in == IN_BF16 || in == IN_F16) ? 64 : 32; }

const SliceCand* slice_cands(int in, int& n) {
    n = 3;
    if (in == IN_BF16 || in == IN_F16) return SLICE_16;
    return in == IN_F32X3 ? SLICE_X3 : SLICE_F32;
}

// Largest output, in 128 x 128 tiles, that takes slice-K: for fp32 up to 144
// (1536^2; at 1024 x 2048 x 1024 44 against 67 us for the grid, at 1536^3 79
// against 98 us; at 2048^2 x 1024 the grid is faster, 69 against 89 us); for
// 3 x bf16, whose grid kernel is five times faster per tile, up to 64 (at 128
// and 144 tiles the two were within 10 % either way); for bf16 / fp16 up to
// 64 (at 128 tiles the grid was faster, 11.8 against 14.8 us at
// 1024 x 2048 x 1024).
int64_t slice_max_tiles128(int in) { return in == IN_F32 ? 144 : 64; }

bool slice_eligible(int in, int M, int N) {
    return slice_format(in) && M > 0 && N > 0 &&
           ceil_div(M, 128) * ceil_div(N, 128) <= slice_max_tiles128(in);
}

int64_t slice_per_cu(const SliceCand& c, int M, int N) {
    return ceil_div(ceil_div(M, c.ts) * ceil_div(N, c.ts), NUM_CU);
}

double slice_load(const SliceCand& c, int64_t n) { return n == 1 ? 1.0 : (double)n * c.co; }

// Cost per block of K of one wave, at the grid's fill of the CUs.
double slice_blk(const SliceCand& c, int M, int N) {
    const int64_t tiles = ceil_div(M, c.ts) * ceil_div(N, c.ts);
    const double fill = tiles >= NUM_CU ? 1.0 : (double)tiles / NUM_CU;
    return c.blk_us + c.fill_us * fill;
}

double estimate_slice_us(int in, const SliceCand& c, int M, int N, int K) {
    const int64_t n = slice_per_cu(c, M, N);
    const int64_t nbw = ceil_div(ceil_div(K, slice_bk(in)), c.waves);
    return c.fixed_us + (double)nbw * slice_blk(c, M, N) * slice_load(c, n) +
           (double)(n - 1) * c.round_us;
}

// The candidate of format `in` with tile ts and `waves` waves (nullptr: none).
const SliceCand* slice_cand(int in, int ts, int waves) {
    int n = 0;
    const SliceCand* c = slice_cands(in, n);
    for (int i = 0; i < n; ++i)
        if (c[i].ts == ts && c[i].waves == waves) return &c[i];
    return nullptr;
}

// The slice-K tile for M x N (32 or 64): the smaller cost per block of K of
// the 4-wave candidates.  It depends on M and N only, so that dgemm_tile_map
// stays exact.
int slice_tile(int in, int M, int N) {
    const SliceCand& c32 = *slice_cand(in, 32, 4);
    const SliceCand& c64 = *slice_cand(in, 64, 4);
    return slice_blk(c32, M, N) * slice_load(c32, slice_per_cu(c32, M, N)) <=
                   slice_blk(c64, M, N) * slice_load(c64, slice_per_cu(c64, M, N))
               ? 32
               : 64;
}

// Waves per workgroup for tile ts: the faster estimate among the format's
// candidates of that tile.
int slice_waves(int in, int ts, int M, int N, int K) {
    int n = 0;
    const SliceCand* c = slice_cands(in, n);
    int best = 0;
    double best_us = 0.0;
    for (int i = 0; i < n; ++i) {
        if (c[i].ts != ts) continue;
        const double us = estimate_slice_us(in, c[i], M, N, K);
        if (best == 0 || us < best_us) { best = c[i].waves; best_us = us; }
    }
    return best;
}

Plan slice_plan(int in, int M, int N, int K) {
    const int ts = slice_tile(in, M, N);
    Plan p{ts, ts, 1, K, 0, 0};
    p.waves = slice_waves(in, ts, M, N, K);
    return p;
}

// Unsplit macro-tile choice: minimise rounds(tiles) x area / eff.  It depends
// on M, N and the input format only, so the host query reports exactly what
// an unsplit launch uses.
TileCand pick_tile(int in, int M, int N) {
    if (slice_eligible(in, M, N)) {
        const int ts = slice_tile(in, M, N);
        return TileCand{ts, ts, 1.0, 0.0, 0.0, 1.0, 1.0};
    }
    int n = 0;
    const TileCand* cands = tiles_for(in, n);
    TileCand best = cands[0];
    double best_cost = -1.0;
    for (int i = 0; i < n; ++i) {
        const TileCand& c = cands[i];
        const int64_t tiles = ceil_div(M, c.bm) * ceil_div(N, c.bn);
        const double cost = rounds_factor(c, tiles, true) * c.bm * c.bn / tile_eff(c, tiles);
        if (best_cost < 0 || cost < best_cost) { best_cost = cost; best = c; }
    }
    return best;
}

double estimate_us(int in, int es_out, int M, int N, const TileCand& t, int splits,
                   int steps_per_split, int ldw) {
    const int64_t tiles = ceil_div(M, t.bm) * ceil_div(N, t.bn);
    const int64_t wgs = tiles * splits;
    double us = rounds_factor(t, wgs) *
                (steps_per_split * step_us(in) * t.bm * t.bn / 65536.0 / tile_eff(t, wgs) +
                 WG_FIXED_US);
    if (splits > 1)
        us += REDUCE_FIXED_US + (2.0 * splits * M * (double)ldw * 4 + (double)M * N * es_out) /
                                    HBM_BYTES_PER_US;
    return us;
}

// ------------------------------------------------------------------ Stream-K
//
// The nine-levels tutorial's section 2.9 puts Stream-K beside Split-K: every
// workgroup gets the same number of K steps, whatever the tile count, so no
// CU idles.  Here (dgemm_internal.h has the schedule): for grids of at most
// one 256 x 256 tile per CU, a persistent grid of one workgroup per CU, each
// computing an equal run of 64-k steps across tile boundaries, then reducing
// its share of each tile it touched.  Estimated time, fitted to measurements
// of the kernel (bf16, MI355X, eight shapes from 512 x 4096 x 4096 to
// 3840 x 3840 x 8192):
//
//   SK_FIXED_US + q * step_us * (aligned ? 1 : SK_UNALIGNED)
//
// with q = the steps of the longest run.  SK_FIXED_US is mostly the fp32
// partial tiles' round trip: every workgroup writes at least one 256 KiB
// tile and its share of the reduction reads as much back, 64-128 MiB in all,
// more than the XCDs' L2s hold.  When the runs do not start on tile
// boundaries (a whole number of workgroups per tile), the 32 workgroups of an
// XCD work at unrelated k offsets of different tiles, and the A and B panels
// they load are no longer shared through L2 as in the grid plans, where an
// XCD's tiles advance through k together: each step then costs SK_UNALIGNED
// times as much.  Stream-K is chosen over the best grid plan (split or not)
// when predicted SK_MARGIN faster -- on the shapes measured, never -- and
// never while the stream is being captured into a graph: each launch tags its
// partials with a fresh 64-bit value from the host, which a replayed graph
// would repeat.

constexpr double SK_FIXED_US = 33.0;
constexpr double SK_UNALIGNED = 1.45;
constexpr double SK_MARGIN = 0.95;

// Whether the Stream-K kernel can run this problem: 16-bit inputs, at least
// one K step, at most one tile per CU (so no XCD has more tiles than ranks),
// and at least one iteration per rank on every XCD with a tile (an XCD gets
// floor or ceil of tiles / 8 of them).
bool sk_feasible(int in, int M, int N, int K) {
    if (!(in == IN_BF16 || in == IN_F16) || K <= 0 || M <= 0 || N <= 0) return false;
    const int64_t nk = ceil_div(K, SK_BK);
    const int64_t tiles = ceil_div(M, SK_TILE) * ceil_div(N, SK_TILE);
    const int64_t nx_min = std::max<int64_t>(1, tiles / NUM_XCD);
    return tiles <= NUM_CU && nk < ((int64_t)1 << 24) && nx_min * nk >= NUM_CU / NUM_XCD;
}

double estimate_sk_us(int in, int M, int N, int K) {
    const int64_t nk = ceil_div(K, SK_BK);
    const int64_t tiles = ceil_div(M, SK_TILE) * ceil_div(N, SK_TILE);
    const int64_t R = NUM_CU / NUM_XCD;
    const int64_t nx = ceil_div(tiles, NUM_XCD);
    const bool aligned = tiles % NUM_XCD == 0 && R % nx == 0;
    const double q = (double)ceil_div(nx * nk, R);
    return SK_FIXED_US + q * step_us(in) * (aligned ? 1.0 : SK_UNALIGNED);
}

Plan sk_plan(int M, int N, int K) {
    Plan p{SK_TILE, SK_TILE, 1, K, 0, sk_ws_bytes(NUM_CU)};
    p.kind = PLAN_STREAM_K;
    (void)M;
    (void)N;
    return p;
}

// Plan choice forced by dgemm_set_plan_override (tests and tuning).
std::atomic<int> g_override_kind{DGEMM_PLAN_AUTO};
std::atomic<int> g_override_bm{0}, g_override_bn{0}, g_override_splits{1};

Plan make_plan_auto(int in, int es_out, int M, int N, int K, uint64_t ws_avail, bool allow_sk) {
    const bool slice = slice_eligible(in, M, N);
    const TileCand base = pick_tile(in, M, N);
    Plan plan = slice ? slice_plan(in, M, N, K) : Plan{base.bm, base.bn, 1, K, 0, 0};
    if (ws_avail == 0 || K == 0 || M == 0 || N == 0) return plan;
    const int bk = bk_of(in);
    const int nk = (int)ceil_div(K, bk);
    const int ldw = (int)ceil_div(N, 4) * 4;
    double best = (slice ? estimate_slice_us(in, *slice_cand(in, plan.bm, plan.waves), M, N, K)
                         : estimate_us(in, es_out, M, N, base, 1, nk, ldw)) *
                  SPLIT_MARGIN;
    int ncand = 0;
    const TileCand* cands = tiles_for(in, ncand);
    for (int c = 0; c < ncand; ++c) {
        for (int s = 2; s <= MAX_SPLITS && s <= nk; ++s) {
            const int steps = (int)ceil_div(nk, s);
            if (ceil_div(nk, steps) != s) continue;  // same work as a smaller s
            const int64_t tiles = ceil_div(M, cands[c].bm) * ceil_div(N, cands[c].bn);
            if (tiles * s > INT32_MAX) continue;
            const int64_t ws = (int64_t)s * M * ldw * 4;
            if ((uint64_t)ws > ws_avail) continue;
            if ((int64_t)PANEL_ROWS * ldw * 4 >= DESC_LIMIT) continue;  // partials' panel limit
            const double us = estimate_us(in, es_out, M, N, cands[c], s, steps, ldw);
            if (us < best) {
                best = us;
                plan = Plan{cands[c].bm, cands[c].bn, s, steps * bk, ldw, ws};
            }
        }
    }
    if (allow_sk && sk_feasible(in, M, N, K) && (uint64_t)sk_ws_bytes(NUM_CU) <= ws_avail &&
        estimate_sk_us(in, M, N, K) < best * SK_MARGIN)
        plan = sk_plan(M, N, K);
    return plan;
}

// The plan of a call: the override when one is set and this call can take
// it, else the estimate's choice.
Plan make_plan(int in, int es_out, int M, int N, int K, uint64_t ws_avail, bool allow_sk) {
    const int kind = g_override_kind.load(std::memory_order_relaxed);
    if (kind == DGEMM_PLAN_STREAM_K && allow_sk && sk_feasible(in, M, N, K) &&
        (uint64_t)sk_ws_bytes(NUM_CU) <= ws_avail)
        return sk_plan(M, N, K);
    if (kind == DGEMM_PLAN_GRID && M > 0 && N > 0) {
        const int bm = g_override_bm.load(std::memory_order_relaxed);
        const int bn = g_override_bn.load(std::memory_order_relaxed);
        const int ov_splits = g_override_splits.load(std::memory_order_relaxed);
        // fp32 and 3 x bf16 slice-K tiles: `splits` names the waves per
        // workgroup (1: the planner's count)
        if (slice_format(in) && bm == bn && (bm == 32 || bm == 64) &&
            ceil_div(M, bm) * ceil_div(N, bm) <= INT32_MAX) {
            const int waves = ov_splits == 1 ? slice_waves(in, bm, M, N, K) : ov_splits;
            if (slice_cand(in, bm, waves)) {
                Plan p{bm, bn, 1, K, 0, 0};
                p.waves = waves;
                return p;
            }
        }
        int n = 0;
        const TileCand* cands = tiles_for(in, n);
        for (int c = 0; c < n; ++c) {
            if (cands[c].bm != bm || cands[c].bn != bn) continue;
            const int bk = bk_of(in);
            const int nk = (int)std::max<int64_t>(ceil_div(K, bk), 1);
            const int s = std::min(ov_splits, nk);
            const int steps = (int)ceil_div(nk, s);
            const int splits = (int)ceil_div(nk, steps);
            const int ldw = (int)ceil_div(N, 4) * 4;
            const int64_t ws = splits > 1 ? (int64_t)splits * M * ldw * 4 : 0;
            if (splits > 1 && ((uint64_t)ws > ws_avail || K == 0 ||
                               (int64_t)PANEL_ROWS * ldw * 4 >= DESC_LIMIT ||
                               ceil_div(M, bm) * ceil_div(N, bn) * splits > INT32_MAX))
                break;
            return splits > 1 ? Plan{bm, bn, splits, steps * bk, ldw, ws} : Plan{bm, bn, 1, K, 0, 0};
        }
    }
    return make_plan_auto(in, es_out, M, N, K, ws_avail, allow_sk && kind != DGEMM_PLAN_NO_STREAM_K);
}

// Stream-K launches tag their partials with a value no earlier launch used:
// a process-wide counter from a start drawn from the clock and an address, so
// that flags another process left in a reused buffer are not taken either.
std::atomic<unsigned long long> g_sk_epoch{
    ((unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count() *
     0x9E3779B97F4A7C15ull) ^ (unsigned long long)(uintptr_t)&g_override_kind};

std::atomic<double> g_sk_wait_us{-1.0};  // < 0: from the estimate
std::atomic<int> g_wall_khz[256];        // wall-clock rate per device (0: not yet read)

// Longest wait of a reducing workgroup for the other contributors' pieces of
// a tile, in wall-clock ticks: by default twice the estimated kernel time plus
// 100 us (a piece is normally long done by then; only a grid that is not
// co-resident misses it, and the reducer then computes it itself).
long long sk_wait_ticks(double est_us) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 256) dev = 0;
    int khz = g_wall_khz[dev].load(std::memory_order_relaxed);
    if (khz <= 0) {
        if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess ||
            khz <= 0)
            khz = 100000;  // 100 MHz, the MI300-series constant clock
        g_wall_khz[dev].store(khz, std::memory_order_relaxed);
    }
    double us = g_sk_wait_us.load(std::memory_order_relaxed);
    if (us < 0.0) us = 2.0 * est_us + 100.0;
    return (long long)(us * khz / 1000.0);
}

// Whether `stream` is being captured into a graph (or the query fails).
bool capturing(hipStream_t stream) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &st) != hipSuccess) return true;
    return st != hipStreamCaptureStatusNone;
}

bool epi_needed(const EpiArgs& e) {
    return e.alpha != 1.0f || e.beta != 0.0f || e.bias != nullptr || e.relu != 0;
}

hipError_t launch_family(const GemmLaunch& L) {
    if (L.in == IN_BF16 || L.in == IN_F16)
        return L.slice_waves > 0 ? launch_slicek16(L) : launch_gemm16(L);
    return launch_gemm32(L);
}

// Validated arguments and a plan -> one GEMM launch, a split GEMM into the
// workspace followed by the reduction, or a Stream-K launch.
int run(int in, int outfmt, int M, int N, int K, const void* A, int lda, const void* B, int ldb,
        void* C, int ldc, const EpiArgs& e, const Plan& p, void* ws, hipStream_t stream) {
    GemmLaunch L{};
    L.in = in;
    L.tbm = p.bm;
    L.tbn = p.bn;
    L.A = (const char*)A;
    L.B = (const char*)B;
    L.M = M;
    L.N = N;
    L.K = K;
    L.lda = lda;
    L.ldb = ldb;
    L.tiles_m = (int)ceil_div(M, p.bm);
    L.tiles_n = (int)ceil_div(N, p.bn);
    if ((int64_t)L.tiles_m * L.tiles_n > INT32_MAX) return DGEMM_ERR_TOO_LARGE;
    L.stream = stream;
    // The 16-bit 128 x 128 tile: two workgroups share a CU with a 2-stage ring
    // (64 KiB of LDS each); when the grid has no more workgroups than CUs there is
    // no second one to hide load latency, and a 4-stage ring (128 KiB, loads
    // issued three steps ahead) measured 17-27 % faster.
    const int64_t wgs = (int64_t)L.tiles_m * L.tiles_n * p.splits;
    L.stages = (p.bm == 128 && (in == IN_BF16 || in == IN_F16) && wgs <= NUM_CU) ? 4 : 2;
    L.slice_waves = p.waves;
    if (p.kind == PLAN_STREAM_K) {
        L.out = outfmt;
        L.epi = epi_needed(e);
        L.C = (char*)C;
        L.ldc = ldc;
        L.splits = 1;
        L.kchunk = K;
        L.e = e;
        SkSched s{};
        s.tiles_m = L.tiles_m;
        s.tiles_n = L.tiles_n;
        s.nk = (int)ceil_div(K, SK_BK);
        s.part = (char*)ws;
        s.flags = (unsigned long long*)((char*)ws + sk_ws_bytes(NUM_CU) - (int64_t)NUM_CU * 8);
        s.epoch = g_sk_epoch.fetch_add(1, std::memory_order_relaxed);
        s.wait_ticks = sk_wait_ticks(estimate_sk_us(in, M, N, K));
        return launch_gemm16_sk(L, s, NUM_CU) == hipSuccess ? DGEMM_OK : DGEMM_ERR_LAUNCH;
    }
    if (p.splits == 1) {
        L.out = outfmt;
        L.epi = epi_needed(e);
        L.C = (char*)C;
        L.ldc = ldc;
        L.splits = 1;
        L.kchunk = K;
        L.c_zstride = 0;
        L.e = e;
        return launch_family(L) == hipSuccess ? DGEMM_OK : DGEMM_ERR_LAUNCH;
    }
    L.out = OUT_F32;
    L.epi = false;
    L.C = (char*)ws;
    L.ldc = p.ldw;
    L.splits = p.splits;
    L.kchunk = p.kchunk;
    L.c_zstride = (int64_t)M * p.ldw * 4;
    L.e = EpiArgs{1.0f, 0.0f, nullptr, 0};
    if (launch_family(L) != hipSuccess) return DGEMM_ERR_LAUNCH;
    const hipError_t r = launch_splitk_reduce((const float*)ws, p.splits, (int64_t)M * p.ldw, p.ldw,
                                              (char*)C, ldc, M, N, outfmt, epi_needed(e), e, stream);
    return r == hipSuccess ? DGEMM_OK : DGEMM_ERR_LAUNCH;
}

int out_format(int in, int out) {
    if (out != DGEMM_OUT_F32 && out != DGEMM_OUT_SAME) return -1;
    if (out == DGEMM_OUT_F32 || in == IN_F32 || in == IN_F32X3) return OUT_F32;
    return in == IN_BF16 ? OUT_BF16 : OUT_F16;
}

// The plain entry points: no epilogue, no workspace.  For fp32 inputs `out`
// must be DGEMM_OUT_F32.
int gemm_plain(int in, int M, int N, int K, const void* A, int lda, const void* B, int ldb, void* C,
               int ldc, int out, void* stream) {
    if ((in == IN_F32 || in == IN_F32X3) && out != DGEMM_OUT_F32) return DGEMM_ERR_INVALID_VALUE;
    const int of = out_format(in, out);
    if (of < 0) return DGEMM_ERR_INVALID_VALUE;
    int st = validate(M, N, K, A, lda, B, ldb, C, ldc, in, out_esize(of));
    if (st != DGEMM_OK) return st;
    if (M == 0 || N == 0) return DGEMM_OK;
    st = check_device();
    if (st != DGEMM_OK) return st;
    const Plan p = make_plan_auto(in, out_esize(of), M, N, K, 0, false);
    return run(in, of, M, N, K, A, lda, B, ldb, C, ldc, EpiArgs{1.0f, 0.0f, nullptr, 0}, p, nullptr,
               (hipStream_t)stream);
}

// Device memory of gemm_ex_static's split-K partials: one array on every GPU
// the library runs on, kept until the process ends.  Host code never passes
// `scratch` itself to a kernel (on the host it names a stand-in, not device
// memory); it passes the address hipGetSymbolAddress returns for the current
// device, taken once per device.
static __device__ __align__(256) char scratch[DGEMM_STATIC_SCRATCH_BYTES];

std::mutex g_scratch_mutex;
std::atomic<void*> g_scratch_ptr[256];

// The current device's copy of `scratch`, or DGEMM_ERR_DEVICE.
int static_scratch(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 256) return DGEMM_ERR_DEVICE;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
                return DGEMM_ERR_DEVICE;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return DGEMM_OK;
}

// gemm_ex's checks, plan and launch.  With `use_static`, the workspace is the
// static scratch array (workspace_bytes of it), which no caller buffer can
// overlap.
int gemm_ex_impl(int in, int out, int M, int N, int K, const void* A, int lda, const void* B,
                 int ldb, void* C, int ldc, float alpha, float beta, const float* bias, int act,
                 void* workspace, size_t workspace_bytes, void* stream, bool use_static) {
    if (in < IN_F32 || in > IN_F32X3) return DGEMM_ERR_INVALID_VALUE;
    const int of = out_format(in, out);
    if (of < 0 || (act != DGEMM_ACT_NONE && act != DGEMM_ACT_RELU)) return DGEMM_ERR_INVALID_VALUE;
    if (!use_static && workspace_bytes > 0 && !workspace) return DGEMM_ERR_INVALID_VALUE;
    const int es_out = out_esize(of);
    int st = validate(M, N, K, A, lda, B, ldb, C, ldc, in, es_out);
    if (st != DGEMM_OK) return st;
    if (M == 0 || N == 0) return DGEMM_OK;
    if (bias && ((uintptr_t)bias & 3)) return DGEMM_ERR_MISALIGNED;
    if (!use_static && workspace_bytes > 0 && ((uintptr_t)workspace & 15))
        return DGEMM_ERR_MISALIGNED;
    const Span c = matrix_span(C, M, N, ldc, es_out);
    const Span b = matrix_span(bias, 1, N, N, 4);
    if (bias && spans_overlap(c, b)) return DGEMM_ERR_ALIAS;
    const bool allow_sk = !capturing((hipStream_t)stream);
    const Plan p =
        make_plan(in, es_out, M, N, K, (use_static || workspace) ? workspace_bytes : 0, allow_sk);
    if (p.ws_bytes > 0 && !use_static) {
        const int es = in_esize(in);
        const Span w = matrix_span(workspace, 1, p.ws_bytes, p.ws_bytes, 1);
        if (spans_overlap(w, c) || spans_overlap(w, matrix_span(A, M, K, lda, es)) ||
            spans_overlap(w, matrix_span(B, K, N, ldb, es)) || (bias && spans_overlap(w, b)))
            return DGEMM_ERR_ALIAS;
    }
    st = check_device();
    if (st != DGEMM_OK) return st;
    if (use_static) {
        if (p.ws_bytes > 0) {
            st = static_scratch(&workspace);
            if (st != DGEMM_OK) return st;
        } else {
            workspace = nullptr;
            workspace_bytes = 0;
        }
    }
    return run(in, of, M, N, K, A, lda, B, ldb, C, ldc, EpiArgs{alpha, beta, bias, act}, p, workspace,
               (hipStream_t)stream);
}

}  // namespace
}  // namespace dgemm

using namespace dgemm;

extern "C" {

int gemm_f32(int M, int N, int K, const float* A, int lda, const float* B, int ldb, float* C,
             int ldc, void* stream) {
    return gemm_plain(IN_F32, M, N, K, A, lda, B, ldb, C, ldc, DGEMM_OUT_F32, stream);
}

int gemm_f32_3xbf16(int M, int N, int K, const float* A, int lda, const float* B, int ldb,
                    float* C, int ldc, void* stream) {
    return gemm_plain(IN_F32X3, M, N, K, A, lda, B, ldb, C, ldc, DGEMM_OUT_F32, stream);
}

int gemm_bf16(int M, int N, int K, const void* A, int lda, const void* B, int ldb, void* C,
              int ldc, int out, void* stream) {
    return gemm_plain(IN_BF16, M, N, K, A, lda, B, ldb, C, ldc, out, stream);
}

int gemm_f16(int M, int N, int K, const void* A, int lda, const void* B, int ldb, void* C,
             int ldc, int out, void* stream) {
    return gemm_plain(IN_F16, M, N, K, A, lda, B, ldb, C, ldc, out, stream);
}

int gemm_ex(int in, int out, int M, int N, int K, const void* A, int lda, const void* B, int ldb,
            void* C, int ldc, float alpha, float beta, const float* bias, int act,
            void* workspace, size_t workspace_bytes, void* stream) {
    return gemm_ex_impl(in, out, M, N, K, A, lda, B, ldb, C, ldc, alpha, beta, bias, act, workspace,
                        workspace_bytes, stream, false);
}

int gemm_ex_static(int in, int out, int M, int N, int K, const void* A, int lda, const void* B,
                   int ldb, void* C, int ldc, float alpha, float beta, const float* bias, int act,
                   size_t scratch_bytes, void* stream) {
    if (scratch_bytes > DGEMM_STATIC_SCRATCH_BYTES) return DGEMM_ERR_SCRATCH_SIZE;
    return gemm_ex_impl(in, out, M, N, K, A, lda, B, ldb, C, ldc, alpha, beta, bias, act, nullptr,
                        scratch_bytes, stream, true);
}

int gemm_ex_plan(int in, int out, int M, int N, int K, size_t workspace_bytes, int* tile_rows,
                 int* tile_cols, int* splits, size_t* workspace_used) {
    if (in < IN_F32 || in > IN_F32X3 || M < 0 || N < 0 || K < 0) return DGEMM_ERR_INVALID_VALUE;
    const int of = out_format(in, out);
    if (of < 0) return DGEMM_ERR_INVALID_VALUE;
    if (ceil_div(M, 128) * ceil_div(N, 128) > INT32_MAX) return DGEMM_ERR_TOO_LARGE;
    const Plan p = make_plan(in, out_esize(of), M, N, K, workspace_bytes, true);
    if (tile_rows) *tile_rows = p.bm;
    if (tile_cols) *tile_cols = p.bn;
    if (splits) *splits = p.kind == PLAN_STREAM_K ? 0 : p.splits;
    if (workspace_used) *workspace_used = (size_t)p.ws_bytes;
    return DGEMM_OK;
}

int dgemm_set_plan_override(int kind, int tile_rows, int tile_cols, int splits) {
    if (kind != DGEMM_PLAN_AUTO && kind != DGEMM_PLAN_GRID && kind != DGEMM_PLAN_STREAM_K &&
        kind != DGEMM_PLAN_NO_STREAM_K)
        return DGEMM_ERR_INVALID_VALUE;
    if (kind == DGEMM_PLAN_GRID && splits < 1) return DGEMM_ERR_INVALID_VALUE;
    g_override_bm.store(tile_rows, std::memory_order_relaxed);
    g_override_bn.store(tile_cols, std::memory_order_relaxed);
    g_override_splits.store(kind == DGEMM_PLAN_GRID ? splits : 1, std::memory_order_relaxed);
    g_override_kind.store(kind, std::memory_order_relaxed);
    return DGEMM_OK;
}

int dgemm_set_stream_k_wait_us(double us) {
    if (std::isnan(us)) return DGEMM_ERR_INVALID_VALUE;
    g_sk_wait_us.store(us < 0.0 ? -1.0 : us, std::memory_order_relaxed);
    return DGEMM_OK;
}

int dgemm_stream_k_schedule(int in, int M, int N, int K, int wg, int partials_present, int* items,
                            int max_items, int* n_items) {
    if (n_items) *n_items = 0;
    if (M < 0 || N < 0 || K < 0 || max_items < 0 || (max_items > 0 && !items)) return DGEMM_ERR_INVALID_VALUE;
    if (in != DGEMM_IN_BF16 && in != DGEMM_IN_F16) return DGEMM_ERR_INVALID_VALUE;
    if (!sk_feasible(in, M, N, K) || wg < 0 || wg >= NUM_CU) return DGEMM_ERR_INVALID_VALUE;
    const int G = NUM_CU;
    SkSched sk{};
    sk.tiles_m = (int)ceil_div(M, SK_TILE);
    sk.tiles_n = (int)ceil_div(N, SK_TILE);
    sk.nk = (int)ceil_div(K, SK_BK);
    const SkRun r = sk_run(sk, wg, G);
    int n = 0;
    auto put = [&](int role, int u, int kb, int ke, int slot, int lo, int hi) {
        if (n < max_items) {
            int tm, tn;
            map_tile(r.pos(u), sk.tiles_m, sk.tiles_n, tm, tn);
            int* o = items + 10 * n;
            o[0] = role;
            o[1] = tm;
            o[2] = tn;
            o[3] = kb * SK_BK;
            o[4] = ke == sk.nk ? K : ke * SK_BK;
            o[5] = slot;
            o[6] = r.first(u);
            o[7] = r.last(u);
            o[8] = lo;
            o[9] = hi;
        }
        ++n;
    };
    // The kernel's order, with every other contributor's piece published or
    // every one missing.
    int kb, ke, lo, hi;
    for (int pc = 0; pc < r.npieces; ++pc) {
        r.piece(r.j, r.u0 + pc, kb, ke);
        put(DGEMM_SK_PIECE, r.u0 + pc, kb, ke, r.slot(r.j, r.u0 + pc), 0, 0);
    }
    for (int pc = 0; pc < r.npieces; ++pc) {
        const int u = r.u0 + pc;
        if (!partials_present)
            for (int p = r.first(u); p <= r.last(u); ++p) {
                if (p == r.j) continue;
                r.piece(p, u, kb, ke);
                put(DGEMM_SK_RECOMPUTE, u, kb, ke, r.slot(p, u), 0, 0);
            }
        sk_share(r, u, lo, hi);
        put(DGEMM_SK_REDUCE, u, 0, 0, -1, lo, hi);
    }
    if (n_items) *n_items = n;
    return n <= max_items ? DGEMM_OK : DGEMM_ERR_INVALID_VALUE;
}

const char* dgemm_status_string(int status) {
    switch (status) {
    case DGEMM_OK: return "DGEMM_OK";
    case DGEMM_ERR_INVALID_VALUE: return "DGEMM_ERR_INVALID_VALUE: negative size, NULL pointer or bad enum";
    case DGEMM_ERR_LEADING_DIM: return "DGEMM_ERR_LEADING_DIM: a leading dimension is below its row length";
    case DGEMM_ERR_MISALIGNED: return "DGEMM_ERR_MISALIGNED: a pointer or row pitch is not aligned";
    case DGEMM_ERR_ALIAS: return "DGEMM_ERR_ALIAS: an output overlaps an input or the workspace";
    case DGEMM_ERR_TOO_LARGE: return "DGEMM_ERR_TOO_LARGE: a panel exceeds the 32-bit buffer range";
    case DGEMM_ERR_DEVICE: return "DGEMM_ERR_DEVICE: no gfx950 device is current";
    case DGEMM_ERR_LAUNCH: return "DGEMM_ERR_LAUNCH: the kernel launch failed";
    case DGEMM_ERR_SCRATCH_SIZE:
        return "DGEMM_ERR_SCRATCH_SIZE: scratch_bytes exceeds the static scratch array "
               "(DGEMM_STATIC_SCRATCH_BYTES)";
    default: return "DGEMM: unknown status";
    }
}

int dgemm_tile_map(int M, int N, int in, int wg, int* tile_rows, int* tile_cols, int* num_wg,
                   int* tile_m, int* tile_n) {
    if (M < 0 || N < 0 || in < IN_F32 || in > IN_F32X3) return DGEMM_ERR_INVALID_VALUE;
    const TileCand t = pick_tile(in, M, N);
    const int64_t tm_count = ceil_div(M, t.bm);
    const int64_t tn_count = ceil_div(N, t.bn);
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
