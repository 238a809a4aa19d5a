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

// Per kernel family; each returns hipErrorInvalidValue for a combination it
// has no instantiation for.
hipError_t launch_gemm16(const GemmLaunch& L);  // IN_BF16, IN_F16
hipError_t launch_gemm32(const GemmLaunch& L);  // IN_F32, IN_F32X3

// Split-K reduction: C[i][j] = epilogue(sum_{z < splits} W[z][i][j]) with W
// fp32, row pitch ldw (a multiple of 4) and split stride zstride elements.
hipError_t launch_splitk_reduce(const float* W, int splits, int64_t zstride, int ldw, char* C,
                                int ldc, int M, int N, int out, bool epi, const EpiArgs& e,
                                hipStream_t stream);

}  // namespace dgemm
