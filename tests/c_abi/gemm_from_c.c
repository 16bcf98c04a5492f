/*
 * A plain C (C99) caller of libdense_gemm_amd.so: device memory from the HIP
 * runtime, no Python and no torch in the process.  It shows that the C ABI in
 * include/dense_gemm.h is usable on its own.
 *
 *   gemm_from_c IN OUT
 *
 * IN holds one problem: int32 transA, transB, dtype, entry; int64 M, N, K,
 * lda, ldb, ldc, batch, strideA, strideB, strideC; float alpha, beta; int32
 * epilogue, has_bias; then the stored A, B and C0 buffers (and the bias),
 * each as an int64 element count followed by the elements.  entry 0 calls
 * dg_gemm, 1 dg_gemm_ex.  OUT receives the C buffer after the call.  The
 * program also checks a few argument errors (they return before any GPU
 * work).  Exit status 0 on success.
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "dense_gemm.h"

#define HIP_OK(x)                                                                       \
    do {                                                                                \
        hipError_t e_ = (x);                                                            \
        if (e_ != hipSuccess) {                                                         \
            fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));               \
            exit(3);                                                                    \
        }                                                                               \
    } while (0)

static void *read_buffer(FILE *f, int64_t *count, size_t elem)
{
    if (fread(count, sizeof(int64_t), 1, f) != 1) return NULL;
    void *p = malloc((size_t)(*count > 0 ? *count : 1) * elem);
    if (p && *count > 0 && fread(p, elem, (size_t)*count, f) != (size_t)*count) {
        free(p);
        return NULL;
    }
    return p;
}

int main(int argc, char **argv)
{
    if (argc != 3) {
        fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
        return 2;
    }
    FILE *f = fopen(argv[1], "rb");
    if (!f) return 2;
    int32_t hdr[4];
    int64_t dims[10];
    float ab[2];
    int32_t epi[2];
    if (fread(hdr, sizeof hdr, 1, f) != 1 || fread(dims, sizeof dims, 1, f) != 1 ||
        fread(ab, sizeof ab, 1, f) != 1 || fread(epi, sizeof epi, 1, f) != 1)
        return 2;
    const int ta = hdr[0], tb = hdr[1], dtype = hdr[2], entry = hdr[3];
    const int64_t M = dims[0], N = dims[1], K = dims[2], lda = dims[3], ldb = dims[4],
                  ldc = dims[5], batch = dims[6], sA = dims[7], sB = dims[8], sC = dims[9];
    const size_t elem = dtype == DG_F32 ? 4 : 2;
    int64_t na, nb, nc, nbias = 0;
    void *a = read_buffer(f, &na, elem), *b = read_buffer(f, &nb, elem), *c = read_buffer(f, &nc, elem);
    void *bias = epi[1] ? read_buffer(f, &nbias, elem) : NULL;
    fclose(f);
    if (!a || !b || !c || (epi[1] && !bias)) return 2;

    /* argument errors come back as -i before anything touches the GPU */
    if (dg_gemm(7, 0, 1, 1, 1, 1.f, a, 1, b, 1, 0.f, c, 1, dtype, NULL) != -1) return 4;
    if (dg_gemm(0, 0, 4, 4, 4, 1.f, a, 3, b, 4, 0.f, c, 4, dtype, NULL) != -8) return 4;
    if (strncmp(dg_status_string(-8), "invalid", 7) != 0) return 4;
    if (dg_version() < 100) return 4;

    void *dA, *dB, *dC, *dBias = NULL;
    HIP_OK(hipMalloc(&dA, (size_t)na * elem + 16));
    HIP_OK(hipMalloc(&dB, (size_t)nb * elem + 16));
    HIP_OK(hipMalloc(&dC, (size_t)nc * elem + 16));
    HIP_OK(hipMemcpy(dA, a, (size_t)na * elem, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dB, b, (size_t)nb * elem, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dC, c, (size_t)nc * elem, hipMemcpyHostToDevice));
    if (bias) {
        HIP_OK(hipMalloc(&dBias, (size_t)nbias * elem + 16));
        HIP_OK(hipMemcpy(dBias, bias, (size_t)nbias * elem, hipMemcpyHostToDevice));
    }
    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));
    int rc;
    if (entry == 0)
        rc = dg_gemm(ta, tb, M, N, K, ab[0], dA, lda, dB, ldb, ab[1], dC, ldc, dtype, s);
    else
        rc = dg_gemm_ex(ta, tb, M, N, K, ab[0], dA, lda, sA, dB, ldb, sB, ab[1], dC, ldc, sC,
                        batch, dBias, epi[0], dtype, s);
    if (rc != DG_OK) {
        fprintf(stderr, "dense gemm call failed: %d (%s), hip error %d\n", rc, dg_status_string(rc),
                dg_last_hip_error());
        return 5;
    }
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(c, dC, (size_t)nc * elem, hipMemcpyDeviceToHost));
    HIP_OK(hipStreamDestroy(s));
    HIP_OK(hipFree(dA));
    HIP_OK(hipFree(dB));
    HIP_OK(hipFree(dC));
    if (dBias) HIP_OK(hipFree(dBias));
    FILE *o = fopen(argv[2], "wb");
    if (!o || fwrite(c, elem, (size_t)nc, o) != (size_t)nc) return 2;
    fclose(o);
    free(a);
    free(b);
    free(c);
    free(bias);
    printf("ok\n");
    return 0;
}
