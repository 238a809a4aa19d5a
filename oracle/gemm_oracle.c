/*
 * gemm_oracle.c -- the CPU oracle for C = A*B.  TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load or call this file.  It shares no code, header, table or constant with the
 * HIP path, and the HIP path never calls it.
 *
 * What it computes (the plain definition, nothing more):
 *
 *     C64[i][j] = sum_{k=0}^{K-1} A[i][k] * B[k][j]
 *     S  [i][j] = sum_{k=0}^{K-1} |A[i][k] * B[k][j]|
 *
 * A is row-major M x K (row pitch lda elements), B is row-major K x N (row pitch
 * ldb).  This is the indexing of every kernel on the sgemm tf32 page
 * ("[CUDA 优化实战] sgemm tf32 - 超越 cuBLAS", section 2 sgemm_tf32_bt: A read as
 * row*k+col, B as row*n+col) and of the hgemm page (section 1 hgemm_naive).  The
 * nine-levels tutorial ("CUDA GEMM优化九重天", section 2.1 Naive GEMM) names the
 * one-thread-per-element dot product as the version to check everything against,
 * and its section 3.1 checks results with a CPU triple loop; this file is that
 * triple loop.
 *
 * Inputs are the storage bytes the GPU receives (fp32, or bf16 / fp16 bit
 * patterns).  Each value is widened EXACTLY to fp64 (every fp32, bf16 and fp16
 * value is an fp64 value), products and sums are fp64, and each element's sum
 * runs in ascending k.  Threads split rows only, so results do not depend on the
 * thread count.  Built with -ffp-contract=off: no fused multiply-add may change
 * a rounding.
 *
 * oracle_round() rounds fp64 results directly to the output format with
 * round-to-nearest, ties-to-even (the hgemm page converts its fp32 accumulators
 * with round-to-nearest conversions, section 1 and section 4), written from the
 * IEEE-754 definition: scale to the format's quantum at the value's binade,
 * round to an integer with ties to even, overflow to infinity.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F16 = 2 };

/* ---- exact widening to fp64 ------------------------------------------------ */

static double widen_f32(const void* p, long idx) {
    float f;
    memcpy(&f, (const char*)p + 4 * idx, 4);
    return (double)f;
}

/* bf16 is the upper half of an fp32 bit pattern. */
static double widen_bf16(const void* p, long idx) {
    uint16_t h;
    memcpy(&h, (const char*)p + 2 * idx, 2);
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double widen_f16(const void* p, long idx) {
    uint16_t h;
    memcpy(&h, (const char*)p + 2 * idx, 2);
    int sign = h >> 15;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);               /* subnormal: m * 2^-24       */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);   /* (1 + m/2^10) * 2^(e-15)    */
    return sign ? -v : v;
}

typedef double (*widen_fn)(const void*, long);

static widen_fn widen_for(int dtype) {
    switch (dtype) {
    case ORACLE_F32: return widen_f32;
    case ORACLE_BF16: return widen_bf16;
    case ORACLE_F16: return widen_f16;
    default: return 0;
    }
}

int oracle_widen(int dtype, const void* src, double* dst, long n) {
    widen_fn w = widen_for(dtype);
    if (!w || n < 0) return 1;
    for (long i = 0; i < n; ++i) dst[i] = w(src, i);
    return 0;
}

/* ---- direct fp64 -> format rounding (round to nearest, ties to even) ------- */

/* Round x to a binary format with `p` significand bits (implicit bit included),
 * minimum normal exponent `emin` and maximum exponent `emax`.  Returns the
 * rounded value as an fp64 (exactly representable in the target format). */
static double round_format(double x, int p, int emin, int emax) {
    if (isnan(x) || isinf(x) || x == 0.0) return x;
    int e2;
    frexp(fabs(x), &e2);            /* |x| = f * 2^e2, f in [0.5, 1)          */
    int E = e2 - 1;                 /* |x| in [2^E, 2^(E+1))                  */
    if (E < emin) E = emin;         /* below the normal range: fixed quantum  */
    double q = ldexp(1.0, E - (p - 1));      /* spacing of the format at E   */
    double r = nearbyint(x / q) * q;         /* default mode: ties to even   */
    if (fabs(r) >= ldexp(1.0, emax + 1)) return copysign(INFINITY, x);
    return r;
}

static uint16_t encode_bf16(double r) {
    float f = (float)r;             /* exact: r is a bf16 value               */
    uint32_t u;
    memcpy(&u, &f, 4);
    if (isnan(r)) return 0x7fc0;
    return (uint16_t)(u >> 16);
}

static uint16_t encode_f16(double r) {
    if (isnan(r)) return 0x7e00;
    uint16_t sign = signbit(r) ? 0x8000 : 0;
    double a = fabs(r);
    if (isinf(a)) return sign | 0x7c00;
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);
    int E = e2 - 1;
    if (E < -14)                    /* subnormal: a = m * 2^-24               */
        return sign | (uint16_t)ldexp(a, 24);
    uint16_t m = (uint16_t)(ldexp(a, 10 - E) - 1024.0);
    return sign | (uint16_t)((E + 15) << 10) | m;
}

int oracle_round(int dtype, const double* src, void* dst, long n) {
    if (n < 0) return 1;
    for (long i = 0; i < n; ++i) {
        double x = src[i];
        if (dtype == ORACLE_F32) {
            float f = (float)round_format(x, 24, -126, 127);
            memcpy((char*)dst + 4 * i, &f, 4);
        } else if (dtype == ORACLE_BF16) {
            uint16_t b = encode_bf16(round_format(x, 8, -126, 127));
            memcpy((char*)dst + 2 * i, &b, 2);
        } else if (dtype == ORACLE_F16) {
            uint16_t h = encode_f16(round_format(x, 11, -14, 15));
            memcpy((char*)dst + 2 * i, &h, 2);
        } else {
            return 1;
        }
    }
    return 0;
}

/* ---- the triple loop ------------------------------------------------------- */

typedef struct {
    int dtype, N, K;
    const void* A;
    long lda;
    const double* B64;              /* B widened once: K x N, packed          */
    const int64_t* rows;
    long nrows;
    double* C64;
    double* S;
    int tid, nthreads;
    int status;
} oracle_job;

static void* oracle_worker(void* arg) {
    oracle_job* j = (oracle_job*)arg;
    widen_fn w = widen_for(j->dtype);
    double* arow = (double*)malloc(sizeof(double) * (size_t)(j->K > 0 ? j->K : 1));
    double* acc = (double*)malloc(sizeof(double) * (size_t)(j->N > 0 ? j->N : 1));
    double* sacc = (double*)malloc(sizeof(double) * (size_t)(j->N > 0 ? j->N : 1));
    if (!arow || !acc || !sacc) {
        j->status = 2;
        free(arow); free(acc); free(sacc);
        return 0;
    }
    for (long r = j->tid; r < j->nrows; r += j->nthreads) {
        long i = (long)j->rows[r];
        for (int k = 0; k < j->K; ++k) arow[k] = w(j->A, i * j->lda + k);
        for (int c = 0; c < j->N; ++c) { acc[c] = 0.0; sacc[c] = 0.0; }
        for (int k = 0; k < j->K; ++k) {
            const double a = arow[k];
            const double* b = j->B64 + (size_t)k * (size_t)j->N;
            for (int c = 0; c < j->N; ++c) {
                const double p = a * b[c];
                acc[c] += p;
                sacc[c] += fabs(p);
            }
        }
        memcpy(j->C64 + (size_t)r * (size_t)j->N, acc, sizeof(double) * (size_t)j->N);
        memcpy(j->S + (size_t)r * (size_t)j->N, sacc, sizeof(double) * (size_t)j->N);
    }
    free(arow); free(acc); free(sacc);
    return 0;
}

/*
 * Computes rows rows[0..nrows) of C64 and S for an M x N x K product.
 * C64 and S are packed nrows x N (row r holds output row rows[r]).
 * Returns 0 on success, 1 on a bad argument, 2 on allocation failure.
 */
int oracle_gemm_rows(int dtype, int M, int N, int K,
                     const void* A, long lda, const void* B, long ldb,
                     const int64_t* rows, long nrows,
                     double* C64, double* S, int nthreads) {
    if (!widen_for(dtype) || M < 0 || N < 0 || K < 0 || nrows < 0) return 1;
    if (lda < K || ldb < N) return 1;
    for (long r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= M) return 1;
    if (nrows == 0 || N == 0) return 0;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > nrows) nthreads = (int)nrows;

    double* B64 = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1) * (size_t)N);
    if (!B64) return 2;
    widen_fn w = widen_for(dtype);
    for (long k = 0; k < K; ++k)
        for (long c = 0; c < N; ++c) B64[k * N + c] = w(B, k * ldb + c);

    oracle_job* jobs = (oracle_job*)calloc((size_t)nthreads, sizeof(oracle_job));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) { free(B64); free(jobs); free(th); return 2; }
    int status = 0;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = (oracle_job){dtype, N, K, A, lda, B64, rows, nrows, C64, S, t, nthreads, 0};
    }
    int started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&th[t], 0, oracle_worker, &jobs[t]) != 0) {
            jobs[t].status = -1;    /* run it on this thread instead          */
        } else {
            ++started;
        }
    }
    oracle_worker(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) {
        if (jobs[t].status == -1) { jobs[t].status = 0; oracle_worker(&jobs[t]); }
        else pthread_join(th[t], 0);
    }
    (void)started;
    for (int t = 0; t < nthreads; ++t)
        if (jobs[t].status) status = jobs[t].status;
    free(jobs); free(th); free(B64);
    return status;
}
