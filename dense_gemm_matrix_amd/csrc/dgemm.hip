// dgemm.hip -- the C ABI of include/dgemm.h: argument validation, the launch
// plan (macro-tile shape and split-K count) and the kernel launches.  Host
// code only; the kernels live in gemm16.hip (bf16 / fp16), gemm32.hip (fp32,
// and fp32 via 3 x bf16) and splitk.hip (the split-K reduction).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
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
// rounds = ceil(tiles * s / 256) workgroups per CU.  128 x 128 tiles fit two
// workgroups on a CU: two co-resident ones take `pair` times as long as one
// alone (bf16 1.26, fp32 1.5, 3 x bf16 1.22), so for them rounds counts pairs and
// the term in parentheses is multiplied by `pair`.  A grid of at most one
// workgroup per CU uses `eff1` in place of eff: the 16-bit 128 x 128 tile then
// runs with a deeper LDS ring (4 stages), which only fits one workgroup per CU,
// and the 3 x bf16 one is measured faster alone on its CU than its pair factor
// implies.
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
struct TileCand { int bm, bn; double eff, pair, eff1; };
constexpr TileCand TILES16[] = {{256, 256, 1.0, 0.0, 1.0}, {192, 256, 0.95, 0.0, 0.95},
                                {128, 128, 0.6, 1.26, 0.8}};
constexpr TileCand TILES32[] = {{128, 128, 0.85, 1.5, 0.85}};
constexpr TileCand TILES32X3[] = {{256, 256, 1.0, 0.0, 1.0}, {128, 128, 0.5, 1.22, 0.6}};

// Workgroup rounds per CU for `wgs` workgroups, and the time factor of a round.
double rounds_factor(const TileCand& t, int64_t wgs) {
    const int64_t per_cu = (wgs + NUM_CU - 1) / NUM_CU;
    if (t.pair > 0.0 && per_cu >= 2) return (double)((per_cu + 1) / 2) * t.pair;
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

struct Plan {
    int bm, bn;
    int splits, kchunk;   // kchunk: K per split (a multiple of the K step)
    int ldw;              // row pitch of the fp32 partials, in elements
    int64_t ws_bytes;     // workspace the plan uses (0 when unsplit)
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Unsplit macro-tile choice: minimise rounds(tiles) x area / eff.  It depends
// on M, N and the input format only, so the host query reports exactly what
// an unsplit launch uses.
TileCand pick_tile(int in, int M, int N) {
    int n = 0;
    const TileCand* cands = tiles_for(in, n);
    TileCand best = cands[0];
    double best_cost = -1.0;
    for (int i = 0; i < n; ++i) {
        const TileCand& c = cands[i];
        const int64_t tiles = ceil_div(M, c.bm) * ceil_div(N, c.bn);
        const double cost = rounds_factor(c, tiles) * c.bm * c.bn / tile_eff(c, tiles);
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

Plan make_plan(int in, int es_out, int M, int N, int K, uint64_t ws_avail) {
    const TileCand base = pick_tile(in, M, N);
    Plan plan{base.bm, base.bn, 1, K, 0, 0};
    if (ws_avail == 0 || K == 0 || M == 0 || N == 0) return plan;
    const int bk = bk_of(in);
    const int nk = (int)ceil_div(K, bk);
    const int ldw = (int)ceil_div(N, 4) * 4;
    double best = estimate_us(in, es_out, M, N, base, 1, nk, ldw) * SPLIT_MARGIN;
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
    return plan;
}

bool epi_needed(const EpiArgs& e) {
    return e.alpha != 1.0f || e.beta != 0.0f || e.bias != nullptr || e.relu != 0;
}

hipError_t launch_family(const GemmLaunch& L) {
    return (L.in == IN_BF16 || L.in == IN_F16) ? launch_gemm16(L) : launch_gemm32(L);
}

// Validated arguments -> one GEMM launch, or a split GEMM into the workspace
// followed by the reduction.
int run(int in, int outfmt, int M, int N, int K, const void* A, int lda, const void* B, int ldb,
        void* C, int ldc, const EpiArgs& e, void* ws, uint64_t ws_bytes, hipStream_t stream) {
    const Plan p = make_plan(in, out_esize(outfmt), M, N, K, ws ? ws_bytes : 0);
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
    return run(in, of, M, N, K, A, lda, B, ldb, C, ldc, EpiArgs{1.0f, 0.0f, nullptr, 0}, nullptr, 0,
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
    const Plan p = make_plan(in, es_out, M, N, K, (use_static || workspace) ? workspace_bytes : 0);
    if (p.splits > 1 && !use_static) {
        const int es = in_esize(in);
        const Span w = matrix_span(workspace, 1, p.ws_bytes, p.ws_bytes, 1);
        if (spans_overlap(w, c) || spans_overlap(w, matrix_span(A, M, K, lda, es)) ||
            spans_overlap(w, matrix_span(B, K, N, ldb, es)) || (bias && spans_overlap(w, b)))
            return DGEMM_ERR_ALIAS;
    }
    st = check_device();
    if (st != DGEMM_OK) return st;
    if (use_static) {
        if (p.splits > 1) {
            st = static_scratch(&workspace);
            if (st != DGEMM_OK) return st;
        } else {
            workspace = nullptr;
            workspace_bytes = 0;
        }
    }
    return run(in, of, M, N, K, A, lda, B, ldb, C, ldc, EpiArgs{alpha, beta, bias, act}, workspace,
               workspace_bytes, (hipStream_t)stream);
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
    const Plan p = make_plan(in, out_esize(of), M, N, K, workspace_bytes);
    if (tile_rows) *tile_rows = p.bm;
    if (tile_cols) *tile_cols = p.bn;
    if (splits) *splits = p.splits;
    if (workspace_used) *workspace_used = (size_t)p.ws_bytes;
    return DGEMM_OK;
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
