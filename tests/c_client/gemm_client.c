/*
 * gemm_client.c -- a plain C program that calls libdgemm through include/dgemm.h
 * with no Python and no torch: HIP runtime calls for device memory and a
 * stream, the library for the product.  The GPU tests run it on files written
 * from the seeded input generators and compare what it writes with the oracle.
 *
 * usage: gemm_client ENTRY OUT M N K A.bin B.bin C.bin [ALPHA RELU]
 *   ENTRY  f32 | f32x3 | bf16 | f16 (the plain entry points) or
 *          ex-f32 | ex-f32x3 | ex-bf16 | ex-f16 (gemm_ex with ALPHA, beta 0,
 *          no bias, RELU 0/1, and the workspace that gemm_ex_plan asks for)
 *   OUT    f32 | same (format of C for 16-bit inputs; fp32 inputs ignore it)
 *   A.bin  M x K elements, B.bin K x N, row-major, no padding; C.bin is written
 *          as M x N elements of C's format.
 * On the device every row pitch is padded to the next multiple of 64 bytes plus
 * 64 (so lda > K, ldb > N, ldc > N), and the gap of each C row is filled with a
 * byte pattern that must survive the call.  Before the product, one call with
 * lda < K checks that an invalid argument is reported (when K > 1).
 * Exit status: 0 ok; 2 the library returned an error; 3 a HIP or file error;
 * 4 the gap of C was written; 5 the invalid call was not reported.
 */
#define __HIP_PLATFORM_AMD__ 1
#include <hip/hip_runtime_api.h>

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "dgemm.h"

#define HIP_OK(x)                                                              \
    do {                                                                       \
        hipError_t e_ = (x);                                                   \
        if (e_ != hipSuccess) {                                                \
            fprintf(stderr, "HIP error %s at %s\n", hipGetErrorString(e_), #x);  \
            exit(3);                                                           \
        }                                                                      \
    } while (0)

static void* read_file(const char* path, size_t bytes) {
    void* p = malloc(bytes ? bytes : 1);
    FILE* f = fopen(path, "rb");
    if (!p || !f || fread(p, 1, bytes, f) != bytes) {
        fprintf(stderr, "cannot read %zu bytes from %s\n", bytes, path);
        exit(3);
    }
    fclose(f);
    return p;
}

static size_t padded_pitch(size_t row_bytes) { return (row_bytes + 63) / 64 * 64 + 64; }

int main(int argc, char** argv) {
    if (argc != 9 && argc != 11) {
        fprintf(stderr, "usage: %s ENTRY OUT M N K A.bin B.bin C.bin [ALPHA RELU]\n", argv[0]);
        return 3;
    }
    const char* entry = argv[1];
    const int ex = strncmp(entry, "ex-", 3) == 0;
    const char* fmt = ex ? entry + 3 : entry;
    const int M = atoi(argv[3]), N = atoi(argv[4]), K = atoi(argv[5]);
    const float alpha = argc == 11 ? (float)atof(argv[9]) : 1.0f;
    const int relu = argc == 11 ? atoi(argv[10]) : 0;
    int in;
    if (!strcmp(fmt, "f32")) in = DGEMM_IN_F32;
    else if (!strcmp(fmt, "f32x3")) in = DGEMM_IN_F32_3XBF16;
    else if (!strcmp(fmt, "bf16")) in = DGEMM_IN_BF16;
    else if (!strcmp(fmt, "f16")) in = DGEMM_IN_F16;
    else { fprintf(stderr, "bad ENTRY %s\n", entry); return 3; }
    const size_t es = (in == DGEMM_IN_BF16 || in == DGEMM_IN_F16) ? 2 : 4;
    const int out = (es == 2 && !strcmp(argv[2], "same")) ? DGEMM_OUT_SAME : DGEMM_OUT_F32;
    const size_t esc = out == DGEMM_OUT_SAME ? 2 : 4;

    void* hA = read_file(argv[6], (size_t)M * K * es);
    void* hB = read_file(argv[7], (size_t)K * N * es);
    const size_t pa = padded_pitch((size_t)K * es), pb = padded_pitch((size_t)N * es);
    const size_t pc = padded_pitch((size_t)N * esc);
    const int lda = (int)(pa / es), ldb = (int)(pb / es), ldc = (int)(pc / esc);

    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));
    void *dA, *dB, *dC;
    HIP_OK(hipMalloc(&dA, pa * (M ? M : 1)));
    HIP_OK(hipMalloc(&dB, pb * (K ? K : 1)));
    HIP_OK(hipMalloc(&dC, pc * (M ? M : 1)));
    if (M && K) HIP_OK(hipMemcpy2D(dA, pa, hA, (size_t)K * es, (size_t)K * es, M, hipMemcpyHostToDevice));
    if (K && N) HIP_OK(hipMemcpy2D(dB, pb, hB, (size_t)N * es, (size_t)N * es, K, hipMemcpyHostToDevice));
    HIP_OK(hipMemset(dC, 0x5a, pc * (M ? M : 1)));

    if (K > 1) {
        const int bad = ex ? gemm_ex(in, out, M, N, K, dA, K - 1, dB, ldb, dC, ldc, alpha, 0.0f,
                                     NULL, relu, NULL, 0, s)
                           : in == DGEMM_IN_BF16 ? gemm_bf16(M, N, K, dA, K - 1, dB, ldb, dC, ldc, out, s)
                           : in == DGEMM_IN_F16 ? gemm_f16(M, N, K, dA, K - 1, dB, ldb, dC, ldc, out, s)
                           : in == DGEMM_IN_F32 ? gemm_f32(M, N, K, dA, K - 1, dB, ldb, dC, ldc, s)
                           : gemm_f32_3xbf16(M, N, K, dA, K - 1, dB, ldb, dC, ldc, s);
        if (bad != DGEMM_ERR_LEADING_DIM) {
            fprintf(stderr, "lda < K returned %d (%s)\n", bad, dgemm_status_string(bad));
            return 5;
        }
    }

    int rc;
    void* ws = NULL;
    size_t ws_used = 0;
    if (ex) {
        int tr = 0, tc = 0, splits = 0;
        rc = gemm_ex_plan(in, out, M, N, K, (size_t)1 << 30, &tr, &tc, &splits, &ws_used);
        if (rc) { fprintf(stderr, "gemm_ex_plan: %s\n", dgemm_status_string(rc)); return 2; }
        if (ws_used) HIP_OK(hipMalloc(&ws, ws_used));
        printf("plan: tile %dx%d, %d split(s), workspace %zu bytes\n", tr, tc, splits, ws_used);
        rc = gemm_ex(in, out, M, N, K, dA, lda, dB, ldb, dC, ldc, alpha, 0.0f, NULL, relu, ws,
                     ws_used, s);
    } else if (in == DGEMM_IN_BF16) {
        rc = gemm_bf16(M, N, K, dA, lda, dB, ldb, dC, ldc, out, s);
    } else if (in == DGEMM_IN_F16) {
        rc = gemm_f16(M, N, K, dA, lda, dB, ldb, dC, ldc, out, s);
    } else if (in == DGEMM_IN_F32) {
        rc = gemm_f32(M, N, K, dA, lda, dB, ldb, dC, ldc, s);
    } else {
        rc = gemm_f32_3xbf16(M, N, K, dA, lda, dB, ldb, dC, ldc, s);
    }
    if (rc) { fprintf(stderr, "%s: %s\n", entry, dgemm_status_string(rc)); return 2; }
    HIP_OK(hipStreamSynchronize(s));

    unsigned char* hC = (unsigned char*)malloc(pc * (M ? M : 1));
    HIP_OK(hipMemcpy(hC, dC, pc * (M ? M : 1), hipMemcpyDeviceToHost));
    for (int i = 0; i < M; ++i)
        for (size_t b = (size_t)N * esc; b < pc; ++b)
            if (hC[(size_t)i * pc + b] != 0x5a) {
                fprintf(stderr, "row %d: gap byte %zu written\n", i, b);
                return 4;
            }
    FILE* f = fopen(argv[8], "wb");
    if (!f) { fprintf(stderr, "cannot write %s\n", argv[8]); return 3; }
    for (int i = 0; i < M; ++i)
        if (fwrite(hC + (size_t)i * pc, 1, (size_t)N * esc, f) != (size_t)N * esc) return 3;
    fclose(f);
    printf("%s %s %dx%dx%d lda %d ldb %d ldc %d: ok\n", entry, out == DGEMM_OUT_SAME ? "same" : "f32",
           M, N, K, lda, ldb, ldc);
    HIP_OK(hipFree(dA));
    HIP_OK(hipFree(dB));
    HIP_OK(hipFree(dC));
    if (ws) HIP_OK(hipFree(ws));
    HIP_OK(hipStreamDestroy(s));
    free(hA); free(hB); free(hC);
    return 0;
}
