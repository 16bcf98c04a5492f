/*
 * CPU oracle for C = alpha * op(A) * op(B) + beta * C0, row-major.
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
 *
 * Precision: every input value (fp32, or fp16 decoded from its bits) is
 * widened exactly to fp64; products of two such values are exact in fp64, and
 * sums accumulate in fp64 in strict increasing k.  Alongside the value the
 * oracle returns absum[i,j] = sum_k |op(A)[i,k] * op(B)[k,j]|, which scales
 * the error bound of the comparison.
 *
 * Readings where the pages are silent:
 *   - op(X) = X stored transposed; ld is the row stride of the stored matrix.
 *   - beta == 0: C0 is not read (NaN/Inf there do not propagate).
 *   - alpha == 0 or K == 0: C = beta*C0; A and B are not read.
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

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_F64 = 2 };

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

static double elem(const void *p, int type, int64_t idx)
{
    switch (type) {
    case ORC_F32: return (double)((const float *)p)[idx];
    case ORC_F16: return oracle_f16_to_f64(((const uint16_t *)p)[idx]);
    default:      return ((const double *)p)[idx];
    }
}

typedef struct {
    int ta, tb;
    int64_t M, N, K;
    double alpha, beta;
    const void *A, *B, *C0;
    int64_t lda, ldb, ldc;
    int tyA, tyB, tyC;
    double *ref, *absum;
    /* point mode */
    int64_t npts;
    const int64_t *pi, *pj;
    int nthreads, tid;
} job_t;

/* op(A)[i,k] and op(B)[k,j] read straight from the stored buffers. */
static inline double opA(const job_t *j, int64_t i, int64_t k)
{
    return j->ta ? elem(j->A, j->tyA, k * j->lda + i) : elem(j->A, j->tyA, i * j->lda + k);
}
static inline double opB(const job_t *j, int64_t k, int64_t c)
{
    return j->tb ? elem(j->B, j->tyB, c * j->ldb + k) : elem(j->B, j->tyB, k * j->ldb + c);
}

static void *rows_worker(void *arg)
{
    const job_t *j = (const job_t *)arg;
    int use_ab = (j->alpha != 0.0) && (j->K > 0);
    double *acc = (double *)calloc((size_t)(j->N ? j->N : 1), sizeof(double));
    double *abs_ = (double *)calloc((size_t)(j->N ? j->N : 1), sizeof(double));
    for (int64_t i = j->tid; i < j->M; i += j->nthreads) {
        memset(acc, 0, sizeof(double) * (size_t)j->N);
        memset(abs_, 0, sizeof(double) * (size_t)j->N);
        if (use_ab) {
            for (int64_t k = 0; k < j->K; ++k) {      /* ikj: k outer, j inner */
                double a = opA(j, i, k);
                for (int64_t c = 0; c < j->N; ++c) {
                    double p = a * opB(j, k, c);
                    acc[c] += p;
                    abs_[c] += fabs(p);
                }
            }
        }
        for (int64_t c = 0; c < j->N; ++c) {
            double r = use_ab ? j->alpha * acc[c] : 0.0;
            if (j->beta != 0.0)
                r += j->beta * elem(j->C0, j->tyC, i * j->ldc + c);
            j->ref[i * j->N + c] = r;
            if (j->absum)
                j->absum[i * j->N + c] = use_ab ? abs_[c] : 0.0;
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
        int64_t i = j->pi[p], c = j->pj[p];
        double acc = 0.0, abs_ = 0.0;
        if (use_ab) {
            for (int64_t k = 0; k < j->K; ++k) {
                double t = opA(j, i, k) * opB(j, k, c);
                acc += t;
                abs_ += fabs(t);
            }
        }
        double r = use_ab ? j->alpha * acc : 0.0;
        if (j->beta != 0.0)
            r += j->beta * elem(j->C0, j->tyC, i * j->ldc + c);
        j->ref[p] = r;
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

/* Dense result: ref and absum (may be NULL) are M x N, row stride N.
 * Element types: 0 = fp32, 1 = fp16 bits, 2 = fp64.  nthreads <= 0 uses every
 * online core.  Returns the thread count used, or a negative value on error. */
int oracle_gemm(int transA, int transB, int64_t M, int64_t N, int64_t K, double alpha,
                const void *A, int64_t lda, int typeA, const void *B, int64_t ldb, int typeB,
                double beta, const void *C0, int64_t ldc, int typeC, double *ref, double *absum,
                int nthreads)
{
    job_t j;
    memset(&j, 0, sizeof(j));
    j.ta = transA; j.tb = transB; j.M = M; j.N = N; j.K = K;
    j.alpha = alpha; j.beta = beta;
    j.A = A; j.B = B; j.C0 = C0; j.lda = lda; j.ldb = ldb; j.ldc = ldc;
    j.tyA = typeA; j.tyB = typeB; j.tyC = typeC;
    j.ref = ref; j.absum = absum; j.nthreads = nthreads;
    if (M <= 0 || N <= 0)
        return 0;
    return run(&j, rows_worker);
}

/* Selected elements only: ref[p], absum[p] for (pi[p], pj[p]), p < npts. */
int oracle_gemm_points(int transA, int transB, int64_t M, int64_t N, int64_t K, double alpha,
                       const void *A, int64_t lda, int typeA, const void *B, int64_t ldb,
                       int typeB, double beta, const void *C0, int64_t ldc, int typeC,
                       int64_t npts, const int64_t *pi, const int64_t *pj, double *ref,
                       double *absum, int nthreads)
{
    job_t j;
    memset(&j, 0, sizeof(j));
    j.ta = transA; j.tb = transB; j.M = M; j.N = N; j.K = K;
    j.alpha = alpha; j.beta = beta;
    j.A = A; j.B = B; j.C0 = C0; j.lda = lda; j.ldb = ldb; j.ldc = ldc;
    j.tyA = typeA; j.tyB = typeB; j.tyC = typeC;
    j.ref = ref; j.absum = absum; j.nthreads = nthreads;
    j.npts = npts; j.pi = pi; j.pj = pj;
    if (npts <= 0)
        return 0;
    return run(&j, points_worker);
}
