/*
 * dgemm.h -- dense GEMM C = A*B on AMD MI355X (gfx950), C ABI.
 *
 * The operation (both pages' kernels and the nine-levels tutorial's naive
 * kernel compute exactly this; see the sgemm tf32 page "[CUDA 优化实战] sgemm
 * tf32 - 超越 cuBLAS" section 2, the hgemm page "[CUDA 优化实战] hgemm - 超越
 * cuBLAS" section 1, and "CUDA GEMM优化九重天" section 2.1):
 *
 *     C[i][j] = sum_{k<K} A[i][k] * B[k][j],   0 <= i < M, 0 <= j < N
 *
 * A is row-major M x K with row pitch lda elements, B is row-major K x N with
 * row pitch ldb, C is row-major M x N with row pitch ldc.  Products are
 * accumulated in fp32 (the pages' matrix instructions all accumulate in fp32).
 * C is overwritten (gemm_ex adds alpha, beta, bias and ReLU).  Elements of C outside the M x N
 * window (the ldc - N gap of each row) are never written.
 *
 * Ownership: A, B and C (and gemm_ex's bias and workspace) are DEVICE pointers
 * owned by the caller, all in the memory of the calling thread's current HIP
 * device, and `stream` belongs to that device; the library launches there and
 * does not check where a pointer lives (a pointer into another GPU's memory is
 * the caller's error and faults like any bad address).  The library allocates
 * no device memory and keeps no pointer after a call returns.
 *
 * Execution: each call validates its arguments, enqueues its kernels (one,
 * or two for a split-K plan of gemm_ex) on `stream` (a hipStream_t; NULL
 * means the default stream) and returns without waiting.  Results are visible
 * once the stream has synchronised.  Calls from different host threads on
 * different streams are independent.
 *
 * Errors: a non-zero status is returned and NOTHING is enqueued when the
 * arguments are invalid; C is left untouched.  The library never aborts and
 * keeps no error state beyond the return value.
 *
 * Preconditions (the tutorial's advice in section 6.5 on 16-byte aligned,
 * row-major operands, which this library makes a rule):
 *   - A, B and C are 16-byte aligned, and every row pitch in bytes
 *     (lda*esize_in, ldb*esize_in, ldc*esize_out) is a multiple of 16;
 *   - lda >= max(1, K), ldb >= max(1, N), ldc >= max(1, N);
 *   - 256 rows of A, 64 rows of 16-bit B (32 of fp32 B) and 256 rows of C,
 *     at their row pitches, each span less than 2 GiB (the kernels address
 *     them with 32-bit buffer offsets): DGEMM_ERR_TOO_LARGE otherwise;
 *   - C's bytes overlap neither A's nor B's.  An operand's bytes are its rows
 *     (row i: row-length elements from base + i * pitch), not the gaps
 *     between them.  Operands with the same row pitch in bytes are compared
 *     row by row, so disjoint column windows of one buffer are accepted;
 *     with different pitches the library compares each operand's first to
 *     last byte, so rows that interleave without sharing a byte are still
 *     reported as DGEMM_ERR_ALIAS.
 * Edge semantics: M == 0 or N == 0 is a no-op; K == 0 writes C = 0 (the empty
 * sum).  Any M, N, K >= 0 is accepted; tiles at the matrix edges read zeros
 * beyond K and never store beyond M or N.
 */
#ifndef DGEMM_H
#define DGEMM_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DGEMM_OK = 0,
    DGEMM_ERR_INVALID_VALUE = 1, /* negative M/N/K, NULL pointer with nonzero extent, bad enum   */
    DGEMM_ERR_LEADING_DIM = 2,   /* lda < max(1,K), ldb < max(1,N) or ldc < max(1,N)           */
    DGEMM_ERR_MISALIGNED = 3,    /* a base pointer or a row pitch in bytes not a multiple of 16
                                    (bias: of 4)                                               */
    DGEMM_ERR_ALIAS = 4,         /* C overlaps A, B or the bias; the workspace overlaps any of them */
    DGEMM_ERR_TOO_LARGE = 5,     /* 256*lda*esize, 128*ldb or 256*ldc*esize_out bytes reach 2 GiB */
    DGEMM_ERR_DEVICE = 6,        /* no current device, or it is not a gfx950                     */
    DGEMM_ERR_LAUNCH = 7,        /* the kernel launch reported an error                          */
    DGEMM_ERR_SCRATCH_SIZE = 8   /* gemm_ex_static: scratch_bytes > DGEMM_STATIC_SCRATCH_BYTES   */
} dgemm_status;

/* Format of C for the 16-bit entry points. */
typedef enum {
    DGEMM_OUT_F32 = 0,  /* C is fp32: the accumulator itself                          */
    DGEMM_OUT_SAME = 1  /* C has the input format, rounded once, to nearest even       */
} dgemm_out;

/*
 * fp32 inputs, fp32 C.  gfx950 has no reduced-precision (xf32) matrix
 * instruction, so products use the full-fp32 matrix instruction
 * v_mfma_f32_32x32x2_f32: the sgemm tf32 page's workload (section 0, M = N =
 * K = 4096 fp32) without its tf32 input truncation.  Outputs of at most 144
 * tiles of 128 x 128 (e.g. 1536 x 1536) run slice-K: 32 x 32 or 64 x 64 tiles
 * whose K is split across the 4 or 8 waves of one workgroup and summed in LDS
 * in wave order, so small products fill the GPU with no workspace; results
 * are deterministic for a given shape.
 */
int gemm_f32(int M, int N, int K,
             const float* A, int lda,
             const float* B, int ldb,
             float* C, int ldc,
             void* stream);

/*
 * fp32 inputs, fp32 C, computed with bf16 matrix instructions: each input is
 * split as x = hi + lo (+ e) with hi = bf16(x), lo = bf16(x - hi), |e| <=
 * 2^-16 |x|, and a*b is taken as hi*hi + hi*lo + lo*hi, accumulated in fp32
 * (three v_mfma_f32_32x32x16_bf16 per product, at 8x the fp32 matrix rate).
 * Per product the relative error is at most about 3 * 2^-16; results stay
 * within 1e-4 * sum_k |a_ik * b_kj| of the exact product.  This is the
 * MI355X counterpart of the sgemm tf32 page's approach (fp32 data on
 * reduced-precision tensor units), more accurate than TF32's 10-bit inputs.
 * Non-finite inputs: a NaN propagates as in gemm_f32, but an infinite x has
 * lo = inf - inf = NaN, so the outputs it reaches are NaN, not infinite (as
 * are those of finite inputs too large for bf16, |x| >= (2 - 2^-8) * 2^127).
 * Outputs of at most 64 tiles of 128 x 128 run slice-K as in gemm_f32.
 * Arguments, layout, errors and execution as gemm_f32.
 */
int gemm_f32_3xbf16(int M, int N, int K,
                    const float* A, int lda,
                    const float* B, int ldb,
                    float* C, int ldc,
                    void* stream);

/*
 * bf16 inputs (raw 16-bit storage), fp32 accumulation, C fp32 (out =
 * DGEMM_OUT_F32) or bf16 (out = DGEMM_OUT_SAME).  The hgemm page's workload
 * (section 0, M = N = K = 4096, bf16 in and out).  Outputs of at most 64
 * tiles of 128 x 128 run slice-K as in gemm_f32 (K split across the waves of
 * one workgroup, summed in LDS in wave order; no workspace).
 */
int gemm_bf16(int M, int N, int K,
              const void* A, int lda,
              const void* B, int ldb,
              void* C, int ldc,
              int out,
              void* stream);

/* fp16 inputs; otherwise as gemm_bf16 (the hgemm page covers both formats). */
int gemm_f16(int M, int N, int K,
             const void* A, int lda,
             const void* B, int ldb,
             void* C, int ldc,
             int out,
             void* stream);

/* Input format codes of gemm_ex, gemm_ex_plan and dgemm_tile_map. */
typedef enum {
    DGEMM_IN_F32 = 0,        /* fp32, full-fp32 matrix instruction (as gemm_f32)     */
    DGEMM_IN_BF16 = 1,       /* bf16 storage (as gemm_bf16)                           */
    DGEMM_IN_F16 = 2,        /* fp16 storage (as gemm_f16)                            */
    DGEMM_IN_F32_3XBF16 = 3  /* fp32 through the 3 x bf16 split (as gemm_f32_3xbf16) */
} dgemm_in;

/* Activation of gemm_ex's epilogue. */
typedef enum {
    DGEMM_ACT_NONE = 0,
    DGEMM_ACT_RELU = 1  /* x < 0 -> 0; NaN passes through */
} dgemm_act;

/*
 * The general entry point: GEMM with a fused epilogue and an optional split-K
 * plan (or slice-K, Stream-K; see below).
 *
 *     C[i][j] := act(alpha * sum_k A[i][k] * B[k][j] + beta * C[i][j] + bias[j])
 *
 * The epilogue is evaluated in fp32 on the fp32 sum and rounded once (to
 * nearest even) to C's format; the old C is read in C's format and only when
 * beta != 0 (so C may hold NaN when beta == 0, as in BLAS).  bias is NULL or
 * a device array of N fp32 values (4-byte aligned).  With alpha = 1, beta = 0,
 * bias = NULL and act = DGEMM_ACT_NONE this is exactly the plain entry point
 * for `in`.  The hgemm page's closing discussion names the library kernel it
 * measures against, a bf16 GEMM with a fused ReLU epilogue; bias and
 * alpha/beta are the usual companions of that epilogue.
 *
 * Split-K (the nine-levels tutorial, section 2.9: K divided into pieces that
 * separate workgroups reduce, joined by a second reduction pass): when the
 * grid of output tiles cannot fill the GPU's 256 CUs (few or thin tiles, deep
 * K), a plan may split K into s pieces.  The GEMM kernel then writes s fp32
 * partial products into `workspace` and a second kernel sums them in a fixed
 * order (ascending piece), applies the epilogue and writes C; results are
 * deterministic for a given (shape, workspace_bytes) and differ from the
 * unsplit plan's only in fp32 summation order.  A split plan is used only if
 * the caller's workspace (device memory, 16-byte aligned, at least
 * workspace_bytes long, not overlapping A, B, C or bias) holds it; with
 * workspace = NULL / workspace_bytes = 0 the call never splits.  The
 * workspace is scratch: its contents before and after the call are
 * unspecified, and calls that share one workspace must be ordered (same
 * stream).  gemm_ex_plan reports the plan and the bytes it uses.
 *
 * Slice-K: small outputs (at most 144 tiles of 128 x 128 for fp32, 64 for the
 * other input formats) run by default on 32 x 32 or 64 x 64 tiles whose K is
 * split across the waves of one workgroup and summed in LDS in wave order:
 * no workspace and no second kernel, deterministic for a given shape.  Offered
 * a workspace, the planner compares this plan with the split plans by their
 * estimated times and takes a split plan only when it is estimated at least
 * 10 % faster: deep K on few tiles and, for bf16 / fp16, outputs that fill the
 * CUs with 64 x 64 tiles at K of about 4096 and more.
 *
 * Stream-K (the nine-levels tutorial, section 2.9: the refinement of Split-K
 * that gives every thread block the same amount of work): for bf16 / fp16
 * inputs with at most 256 tiles of 256 x 256, a plan may instead run one
 * persistent workgroup per CU, each taking an equal run of K steps across
 * tile boundaries; the workgroups that share a tile then reduce it together,
 * each adding up its share of the tile's outputs over their fp32 partial sums
 * (in the workspace) in k order: results are deterministic for a given
 * (shape, workspace_bytes) and differ from the other plans' only in fp32
 * summation order.  It needs 2 x 256 x 256 KiB + 2 KiB of workspace
 * (128 MiB), and is never used on a stream that is being captured into a
 * graph (hipStreamIsCapturing).  A workgroup waits a bounded time for a
 * partial and otherwise computes it itself, so the result does not depend on
 * how the grid is scheduled.  On MI355X it measured slower than the other
 * plans on every shape tried, so the cost model does not pick it; it runs when
 * forced with dgemm_set_plan_override.
 *
 * in:  a dgemm_in code.  out: DGEMM_OUT_F32, or DGEMM_OUT_SAME for C in the
 * input format (for fp32 inputs both mean fp32).  Other arguments,
 * preconditions and errors as the plain entry points.
 */
int gemm_ex(int in, int out, int M, int N, int K,
            const void* A, int lda,
            const void* B, int ldb,
            void* C, int ldc,
            float alpha, float beta, const float* bias, int act,
            void* workspace, size_t workspace_bytes,
            void* stream);

/* Bytes of the static device array that gemm_ex_static uses as its workspace. */
#define DGEMM_STATIC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * gemm_ex for callers that cannot allocate device memory: code being captured
 * into a HIP graph, tight serving loops, harnesses that forbid hipMalloc.  It
 * computes exactly what gemm_ex computes with a workspace of scratch_bytes,
 * and the split-K partials go to a static device array of
 * DGEMM_STATIC_SCRATCH_BYTES (32 MiB) that the library holds on every GPU it
 * runs on until the process ends.  The call allocates nothing; the caller
 * passes A, B, C and bias as for gemm_ex.  scratch_bytes (0 ..
 * DGEMM_STATIC_SCRATCH_BYTES) bounds the plan as gemm_ex's workspace_bytes
 * does: gemm_ex_plan(..., scratch_bytes, ...) reports the plan, and 0 never
 * splits.  A larger value returns DGEMM_ERR_SCRATCH_SIZE before anything is
 * enqueued.  Every call on one GPU shares that GPU's array, and no part of it
 * needs to start at zero (every partial is written before it is read): calls
 * whose kernels overlap in time on one GPU (different streams, or different
 * host threads without ordering) race on it and must be ordered by the
 * caller, e.g. by issuing them on one stream.  The array's address is looked
 * up on a device's first call.
 */
int gemm_ex_static(int in, int out, int M, int N, int K,
                   const void* A, int lda,
                   const void* B, int ldb,
                   void* C, int ldc,
                   float alpha, float beta, const float* bias, int act,
                   size_t scratch_bytes,
                   void* stream);

/*
 * Host-side query of the plan gemm_ex would use with `workspace_bytes`
 * available (no GPU needed): macro-tile shape, split count (1 = unsplit,
 * 0 = a Stream-K plan) and the workspace bytes that plan uses (0 when
 * unsplit).  gemm_ex never takes a Stream-K plan on a stream that is being
 * captured into a graph; this query assumes no capture.  Any output pointer
 * may be NULL.  Returns DGEMM_OK, or DGEMM_ERR_INVALID_VALUE for negative
 * sizes or a bad `in` / `out`.
 */
int gemm_ex_plan(int in, int out, int M, int N, int K, size_t workspace_bytes,
                 int* tile_rows, int* tile_cols, int* splits, size_t* workspace_used);

/* Plan kinds of dgemm_set_plan_override. */
typedef enum {
    DGEMM_PLAN_AUTO = 0,      /* the cost model's choice (the default)                */
    DGEMM_PLAN_GRID = 1,      /* one workgroup per tile and K split, as given         */
    DGEMM_PLAN_STREAM_K = 2,  /* Stream-K (16-bit inputs; 256 x 256 tiles)            */
    DGEMM_PLAN_NO_STREAM_K = 3 /* the cost model's choice among the other plans       */
} dgemm_plan_kind;

/*
 * Process-wide plan override for gemm_ex, gemm_ex_static and gemm_ex_plan,
 * for tests and for tuning the cost model (the plain entry points ignore it).
 * DGEMM_PLAN_GRID forces the macro-tile tile_rows x tile_cols (a shape the
 * input format's kernel has: 256 x 256, 192 x 256 or 128 x 128 for 16-bit
 * inputs, 128 x 128 for fp32, 256 x 256 or 128 x 128 for 3 x bf16) and
 * `splits` K pieces (>= 1; reduced to the number of K steps); it also forces
 * the slice-K tiles, 32 x 32 or 64 x 64 at any M and N in every input format,
 * where `splits` gives the waves per workgroup instead (4 or 8 for 32 x 32, 4
 * for 64 x 64, 1 for the planner's count; a slice-K plan has no K pieces);
 * DGEMM_PLAN_STREAM_K forces a Stream-K plan, DGEMM_PLAN_NO_STREAM_K rules it
 * out (tile and split arguments ignored by both).  A forced plan the call cannot take (tile shape the kernel lacks,
 * workspace too small, Stream-K for fp32 inputs or under graph capture) falls
 * back to the cost model's choice, which gemm_ex_plan then reports.
 * DGEMM_PLAN_AUTO clears the override.  Not synchronised with calls running
 * on other host threads.  Returns DGEMM_OK, or DGEMM_ERR_INVALID_VALUE for a
 * bad kind or splits < 1 with DGEMM_PLAN_GRID.
 */
int dgemm_set_plan_override(int kind, int tile_rows, int tile_cols, int splits);

/*
 * Process-wide bound on how long a Stream-K workgroup waits for another's
 * partial sums before computing them itself, in microseconds; us < 0 restores
 * the default (twice the plan's estimated time plus 100 us), and 0 makes every
 * workgroup take only what is already there (a test of the fallback path,
 * whose results are bit for bit those of the waiting path).  Returns DGEMM_OK,
 * or DGEMM_ERR_INVALID_VALUE for NaN.
 */
int dgemm_set_stream_k_wait_us(double us);

/* Item roles reported by dgemm_stream_k_schedule. */
typedef enum {
    DGEMM_SK_PIECE = 0,      /* the workgroup's own k range of a tile, summed into `slot`   */
    DGEMM_SK_RECOMPUTE = 1,  /* another contributor's missing piece, into that one's slot  */
    DGEMM_SK_REDUCE = 2      /* blocks [lo, hi) of the tile: contributors first .. last
                                summed in that order, epilogue, stored to C             */
} dgemm_sk_role;

/*
 * Host-side query of the Stream-K schedule (no GPU needed; for tests and
 * tuning): the items workgroup `wg` (0 <= wg < 256; XCD x = wg % 8, rank
 * wg / 8) of a Stream-K launch runs for an M x N x K GEMM with 16-bit inputs
 * (`in` = DGEMM_IN_BF16 or DGEMM_IN_F16), in the order it runs them, with
 * every other contributor's piece already published (partials_present != 0)
 * or every one missing (0: the workgroup computes each itself).  Each item is
 * 10 ints in `items`: role (dgemm_sk_role), the tile's row and column index
 * (256 x 256 tiles), k_begin and k_end (elements of K; PIECE and RECOMPUTE),
 * the slot (0 .. 511; slots 2 wg and 2 wg + 1 hold workgroup wg's pieces;
 * -1 for REDUCE), the tile's first and last contributor (ranks of XCD x), and
 * lo and hi (REDUCE: the tile's 32 x 32 output blocks [lo, hi) of 64, block
 * q at rows 128 (q / 32) + 32 ((q / 4) % 4), columns 128 ((q / 16) % 2) +
 * 32 (q % 4) of the tile; 0 otherwise).  *n_items receives the count; only
 * the first max_items are written.  Returns DGEMM_OK, or
 * DGEMM_ERR_INVALID_VALUE for a shape Stream-K does not run (other than 16-bit
 * inputs with at most 256 tiles and at least 32 steps of 64 k per XCD that has
 * a tile), a bad argument, or max_items below the count.
 */
int dgemm_stream_k_schedule(int in, int M, int N, int K, int wg, int partials_present, int* items,
                            int max_items, int* n_items);

/* A static, NUL-terminated description of a status code (never NULL). */
const char* dgemm_status_string(int status);

/*
 * Host-side query of the kernel's work distribution, for tests and tuning; it
 * launches nothing and needs no GPU.  For a problem of M x N outputs and input
 * format `in` (a dgemm_in code), as the plain entry points launch it (no
 * split), writes the macro-tile shape and
 * the number of workgroups, and, when wg is in [0, *num_wg), the output tile
 * (row block *tile_m, column block *tile_n) that workgroup `wg` computes.  The
 * mapping is a bijection from workgroups to tiles: it first gives each of the
 * 8 XCDs a contiguous run of tiles (workgroups are dispatched to XCDs in turn),
 * then walks each run in column strips a few tile rows high so that
 * neighbouring workgroups share A and B panels in L2 (the sgemm tf32 page's
 * "Grid Swizzling", section 4).  Any output pointer may be NULL.
 * Returns DGEMM_OK, or DGEMM_ERR_INVALID_VALUE for negative sizes or a bad `in`.
 */
int dgemm_tile_map(int M, int N, int in, int wg,
                   int* tile_rows, int* tile_cols, int* num_wg,
                   int* tile_m, int* tile_n);

#ifdef __cplusplus
}
#endif

#endif /* DGEMM_H */
