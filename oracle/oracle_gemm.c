/*
 * CPU oracle for C = act(alpha * op(A) * op(B) + beta * C0 + bias), row-major,
 * for one matrix or a strided batch of them.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the independent reference the GPU
 * library is checked against.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark load it.  It shares no source, header,
 * table or helper with the GPU library, and the library never calls it.
 *
 * What it computes (the definition, written out):
 *   - "Optimizing GEMM on Apple's M5 from scratch, Part 1", Introduction: full
 *     SGEMM is C = alpha*A*B + beta*C; the pages' own runs fix alpha=1, beta=0.
 *   - same page, "Kernel 1: Naive Implementation": every C[i,j] is the dot
 *     product of row i of A with column j of B, summed over k = 0..K-1.
 *   - "From a C loop to a GPU kernel", "Two lines swapped, 17x": the ikj loop
 *     order walks B and C along rows while each C element still receives its
 *     terms in increasing k, so it keeps the plain loop's rounding order.
 *   - "Metal GEMM Kernels for LoRA Training on Apple Silicon", section 2: the
 *     transpose variants, A stored [K,M] for "t" and B stored [N,K] for "t".
 *   - "From a C loop to a GPU kernel", "Fusion": a fused GEMM epilogue adds a
 *     learned per-output offset (bias) to the product and applies an
 *     elementwise activation (the page's example is gelu) before the single
 *     write of the result.  Here the output of a row-major C = X W^T is a
 *     column, so bias[j] is added to every element of column j.
 *   - "Metal GEMM Kernels for LoRA Training on Apple Silicon", section 8:
 *     attention's per-head products are the same GEMM variants repeated over
 *     heads at a fixed offset; batch b reads A + b*strideA, B + b*strideB and
 *     C0 + b*strideC (strides in elements, any of them may be 0).
 *
 * Precision: every input value (fp32, or fp16 / bf16 decoded from its bits)
 * is widened exactly to fp64; products of two such values are exact in fp64,
 * and sums accumulate in fp64 in strict increasing k.  Alongside the value the
 * oracle returns absum[i,j] = sum_k |op(A)[i,k] * op(B)[k,j]|, which scales
 * the error bound of the comparison, and optionally the value before the
 * activation, which the bound of an activated output is derived from.
 *
 * Activations (act):
 *   0 none; 1 relu, max(x, 0) (NaN propagates); 2 gelu in its defining form
 *   x * Phi(x) = x/2 * (1 + erf(x / sqrt(2))) (Hendrycks & Gimpel 2016),
 *   Phi being the standard normal distribution function.
 *
 * Readings where the pages are silent:
 *   - op(X) = X stored transposed; ld is the row stride of the stored matrix.
 *   - beta == 0: C0 is not read (NaN/Inf there do not propagate).
 *   - alpha == 0 or K == 0: the product term is 0 and A and B are not read.
 *   - the epilogue order: x = alpha*acc + beta*C0 + bias[j], then act(x).
 *   - bf16: 16-bit patterns, sign bit 15, 8 exponent bits (bias 127), 7
 *     fraction bits (the upper half of an fp32 encoding).
 *
 * Threads: rows of C are split over POSIX threads ("From a C loop to a GPU
 * kernel", "The lever I'd been ignoring: more cores"); each row is computed by
 * one thread, so the result does not depend on the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_F64 = 2, ORC_BF16 = 3 };
enum { ORC_ACT_NONE = 0, ORC_ACT_RELU = 1, ORC_ACT_GELU = 2 };

/* IEEE 754 binary16 -> binary64, from the format's definition:
 * sign bit 15, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);              /* zero or subnormal */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f + 1024), e - 25);  /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16 -> binary64, from the format's definition: sign bit 15, 8
 * exponent bits (bias 127), 7 fraction bits. */
double oracle_bf16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 7) & 0xff;
    int f = h & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);             /* zero or subnormal: f/128 * 2^-126 */
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f + 128), e - 134);  /* (1 + f/128) * 2^(e-127) */
    return sign ? -v : v;
}

static double elem(const void *p, int type, int64_t idx)
{
    switch (type) {
    case ORC_F32:  return (double)((const float *)p)[idx];
    case ORC_F16:  return oracle_f16_to_f64(((const uint16_t *)p)[idx]);
    case ORC_BF16: return oracle_bf16_to_f64(((const uint16_t *)p)[idx]);
    default:       return ((const double *)p)[idx];
    }
}

/* The activation of the epilogue, in fp64. */
static double activation(int act, double x)
{
    switch (act) {
    case ORC_ACT_RELU: return x > 0.0 ? x : (x != x ? x : 0.0);
    case ORC_ACT_GELU: return 0.5 * x * (1.0 + erf(x / sqrt(2.0)));
    default:           return x;
    }
}

typedef struct {
    int ta, tb;
    int64_t M, N, K;
    double alpha, beta;
    const void *A, *B, *C0, *bias;
    int64_t lda, ldb, ldc;
    int64_t sA, sB, sC;       /* batch strides (elements) */
    int64_t batch;
    int tyA, tyB, tyC, tyBias;
    int act;
    double *ref, *pre, *absum;
    /* point mode */
    int64_t npts;
    const int64_t *pb, *pi, *pj;
    int nthreads, tid;
} job_t;

/* op(A)[i,k] and op(B)[k,j] of batch b, read straight from the stored buffers. */
static inline double opA(const job_t *j, int64_t b, int64_t i, int64_t k)
{
    int64_t o = b * j->sA;
    return j->ta ? elem(j->A, j->tyA, o + k * j->lda + i) : elem(j->A, j->tyA, o + i * j->lda + k);
}
static inline double opB(const job_t *j, int64_t b, int64_t k, int64_t c)
{
    int64_t o = b * j->sB;
    return j->tb ? elem(j->B, j->tyB, o + c * j->ldb + k) : elem(j->B, j->tyB, o + k * j->ldb + c);
}

/* The epilogue value before the activation: alpha*acc + beta*C0 + bias[c]. */
static inline double combine(const job_t *j, int use_ab, double acc, int64_t b, int64_t i, int64_t c)
{
    double r = use_ab ? j->alpha * acc : 0.0;
    if (j->beta != 0.0)
        r += j->beta * elem(j->C0, j->tyC, b * j->sC + i * j->ldc + c);
    if (j->bias)
        r += elem(j->bias, j->tyBias, c);
    return r;
}

/* Rows of every batch: global row g is row g % M of batch g / M. */
static void *rows_worker(void *arg)
{
    const job_t *j = (const job_t *)arg;
    int use_ab = (j->alpha != 0.0) && (j->K > 0);
    double *acc = (double *)calloc((size_t)(j->N ? j->N : 1), sizeof(double));
    double *abs_ = (double *)calloc((size_t)(j->N ? j->N : 1), sizeof(double));
    for (int64_t g = j->tid; g < j->batch * j->M; g += j->nthreads) {
        const int64_t b = g / j->M, i = g % j->M;
        memset(acc, 0, sizeof(double) * (size_t)j->N);
        memset(abs_, 0, sizeof(double) * (size_t)j->N);
        if (use_ab) {
            for (int64_t k = 0; k < j->K; ++k) {      /* ikj: k outer, j inner */
                double a = opA(j, b, i, k);
                for (int64_t c = 0; c < j->N; ++c) {
                    double p = a * opB(j, b, k, c);
                    acc[c] += p;
                    abs_[c] += fabs(p);
                }
            }
        }
        for (int64_t c = 0; c < j->N; ++c) {
            const int64_t o = g * j->N + c;
            double r = combine(j, use_ab, acc[c], b, i, c);
            if (j->pre)
                j->pre[o] = r;
            j->ref[o] = activation(j->act, r);
            if (j->absum)
                j->absum[o] = use_ab ? abs_[c] : 0.0;
        }
    }
    free(acc);
    free(abs_);
    return NULL;
}

static void *points_worker(void *arg)
{
    const job_t *j = (const job_t *)arg;
    int use_ab = (j->alpha != 0.0) && (j->K > 0);
    for (int64_t p = j->tid; p < j->npts; p += j->nthreads) {
        int64_t b = j->pb ? j->pb[p] : 0, i = j->pi[p], c = j->pj[p];
        double acc = 0.0, abs_ = 0.0;
        if (use_ab) {
            for (int64_t k = 0; k < j->K; ++k) {
                double t = opA(j, b, i, k) * opB(j, b, k, c);
                acc += t;
                abs_ += fabs(t);
            }
        }
        double r = combine(j, use_ab, acc, b, i, c);
        if (j->pre)
            j->pre[p] = r;
        j->ref[p] = activation(j->act, r);
        if (j->absum)
            j->absum[p] = use_ab ? abs_ : 0.0;
    }
    return NULL;
}

static int run(job_t *base, void *(*fn)(void *))
{
    int nt = base->nthreads;
    if (nt <= 0) {
        long n = sysconf(_SC_NPROCESSORS_ONLN);
        nt = n > 0 ? (int)n : 1;
    }
    base->nthreads = nt;
    job_t *jobs = (job_t *)malloc(sizeof(job_t) * (size_t)nt);
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nt);
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return -1;
    }
    for (int t = 0; t < nt; ++t) {
        jobs[t] = *base;
        jobs[t].tid = t;
        if (pthread_create(&th[t], NULL, fn, &jobs[t]) != 0) {
            for (int u = 0; u < t; ++u)
                pthread_join(th[u], NULL);
            free(jobs);
            free(th);
            return -2;
        }
    }
    for (int t = 0; t < nt; ++t)
        pthread_join(th[t], NULL);
    free(jobs);
    free(th);
    return nt;
}

/* Dense result of a strided batch: ref, pre and absum (pre and absum may be
 * NULL) are batch x M x N, row stride N; pre is the value before the
 * activation.  Element types: 0 = fp32, 1 = fp16 bits, 2 = fp64, 3 = bf16
 * bits; bias (NULL for none) holds N elements of type typeBias.  nthreads <= 0
 * uses every online core.  Returns the thread count used, or a negative value
 * on error. */
int oracle_gemm_ex(int transA, int transB, int64_t M, int64_t N, int64_t K, double alpha,
                   const void *A, int64_t lda, int64_t strideA, int typeA, const void *B,
                   int64_t ldb, int64_t strideB, int typeB, double beta, const void *C0,
                   int64_t ldc, int64_t strideC, int typeC, const void *bias, int typeBias,
                   int act, int64_t batch, double *ref, double *pre, double *absum, int nthreads)
{
    job_t j;
    memset(&j, 0, sizeof(j));
    j.ta = transA; j.tb = transB; j.M = M; j.N = N; j.K = K;
    j.alpha = alpha; j.beta = beta;
    j.A = A; j.B = B; j.C0 = C0; j.bias = bias;
    j.lda = lda; j.ldb = ldb; j.ldc = ldc;
    j.sA = strideA; j.sB = strideB; j.sC = strideC; j.batch = batch;
    j.tyA = typeA; j.tyB = typeB; j.tyC = typeC; j.tyBias = typeBias; j.act = act;
    j.ref = ref; j.pre = pre; j.absum = absum; j.nthreads = nthreads;
    if (M <= 0 || N <= 0 || batch <= 0)
        return 0;
    return run(&j, rows_worker);
}

/* Selected elements only: ref[p], pre[p], absum[p] for element (pi[p], pj[p])
 * of batch pb[p] (pb NULL: batch 0), p < npts. */
int oracle_gemm_points_ex(int transA, int transB, int64_t M, int64_t N, int64_t K, double alpha,
                          const void *A, int64_t lda, int64_t strideA, int typeA, const void *B,
                          int64_t ldb, int64_t strideB, int typeB, double beta, const void *C0,
                          int64_t ldc, int64_t strideC, int typeC, const void *bias, int typeBias,
                          int act, int64_t npts, const int64_t *pb, const int64_t *pi,
                          const int64_t *pj, double *ref, double *pre, double *absum, int nthreads)
{
    job_t j;
    memset(&j, 0, sizeof(j));
    j.ta = transA; j.tb = transB; j.M = M; j.N = N; j.K = K;
    j.alpha = alpha; j.beta = beta;
    j.A = A; j.B = B; j.C0 = C0; j.bias = bias;
    j.lda = lda; j.ldb = ldb; j.ldc = ldc;
    j.sA = strideA; j.sB = strideB; j.sC = strideC; j.batch = 1;
    j.tyA = typeA; j.tyB = typeB; j.tyC = typeC; j.tyBias = typeBias; j.act = act;
    j.ref = ref; j.pre = pre; j.absum = absum; j.nthreads = nthreads;
    j.npts = npts; j.pb = pb; j.pi = pi; j.pj = pj;
    if (npts <= 0)
        return 0;
    return run(&j, points_worker);
}

/* Single matrix, no bias, no activation: ref and absum (may be NULL) are
 * M x N, row stride N. */
int oracle_gemm(int transA, int transB, int64_t M, int64_t N, int64_t K, double alpha,
                const void *A, int64_t lda, int typeA, const void *B, int64_t ldb, int typeB,
                double beta, const void *C0, int64_t ldc, int typeC, double *ref, double *absum,
                int nthreads)
{
    return oracle_gemm_ex(transA, transB, M, N, K, alpha, A, lda, 0, typeA, B, ldb, 0, typeB,
                          beta, C0, ldc, 0, typeC, NULL, ORC_F64, ORC_ACT_NONE, 1, ref, NULL,
                          absum, nthreads);
}

/* Selected elements of a single matrix, no bias, no activation. */
int oracle_gemm_points(int transA, int transB, int64_t M, int64_t N, int64_t K, double alpha,
                       const void *A, int64_t lda, int typeA, const void *B, int64_t ldb,
                       int typeB, double beta, const void *C0, int64_t ldc, int typeC,
                       int64_t npts, const int64_t *pi, const int64_t *pj, double *ref,
                       double *absum, int nthreads)
{
    return oracle_gemm_points_ex(transA, transB, M, N, K, alpha, A, lda, 0, typeA, B, ldb, 0,
                                 typeB, beta, C0, ldc, 0, typeC, NULL, ORC_F64, ORC_ACT_NONE,
                                 npts, NULL, pi, pj, ref, NULL, absum, nthreads);
}
