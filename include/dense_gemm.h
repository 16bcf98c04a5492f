/*
 * dense_gemm.h -- C ABI of libdense_gemm_amd.so, a dense matrix multiply for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (one call):
 *
 *     C = alpha * op(A) * op(B) + beta * C
 *
 * the full SGEMM form given in "Optimizing GEMM on Apple's M5 from scratch,
 * Part 1", Introduction (whose own runs fix alpha = 1, beta = 0), with the
 * transpose variants of "Metal GEMM Kernels for LoRA Training on Apple
 * Silicon", section 2 ("GEMM structure": nn A[M,K] B[K,N], tn A[K,M]^T B[K,N],
 * nt A[M,K] B[N,K]^T; tt is the remaining combination).
 *
 * Layout.  Every matrix is row-major: element (i, j) of a stored matrix X is
 * X[i * ldX + j] (ld = row stride in elements).  op(A) is M x K and op(B) is
 * K x N:
 *   transA = DG_OP_N: A is stored M x K, lda >= max(1, K)
 *   transA = DG_OP_T: A is stored K x M, lda >= max(1, M)
 *   transB = DG_OP_N: B is stored K x N, ldb >= max(1, N)
 *   transB = DG_OP_T: B is stored N x K, ldb >= max(1, K)
 *   C is stored M x N, ldc >= max(1, N).
 * A sub-matrix is passed as a pointer to its first element plus the parent's
 * ld.  Elements outside the logical extents (padding between rows) are never
 * read and never written.
 *
 * Types (dtype):
 *   DG_F32         A, B, C are fp32; products and sums in fp32 on the fp32
 *                  matrix cores (full precision, no reduced-precision inputs).
 *   DG_F16_F32ACC  A, B, C are IEEE fp16; products are accumulated in fp32
 *                  (the fp16 matrix-core path with fp32 accumulators -- "Metal
 *                  GEMM Kernels for LoRA Training", section 1); the result
 *                  alpha*acc + beta*C is formed in fp32 (an fp16 C is widened
 *                  exactly) and rounded once to fp16, round-to-nearest-even,
 *                  overflow to +-Inf.
 *   DG_BF16_F32ACC A, B, C are bfloat16 (8 significant bits, fp32's exponent
 *                  range); as DG_F16_F32ACC otherwise: fp32 accumulation, one
 *                  round-to-nearest-even to bf16 at the end.  The page above
 *                  (section 1) has bf16 emulated on its GPU; gfx950 has a
 *                  native bf16 matrix-core instruction.
 *   DG_F16_F32OUT  A, B are fp16, C is fp32: the fp16 matrix-core path with
 *                  fp32 accumulators, and alpha*acc + beta*C (fp32 C read as
 *                  is) written to C in fp32 with no rounding to fp16 -- the
 *                  fp32-output variant of "Metal GEMM Kernels for LoRA
 *                  Training", section 4 (writing fp32 straight to device
 *                  memory), for callers that keep fp32 results (gradient
 *                  accumulation, a following fp32 reduction).
 *   DG_BF16_F32OUT A, B are bf16, C is fp32; as DG_F16_F32OUT otherwise.
 *   alpha and beta are fp32 for every type.  The bias of dg_gemm_ex has C's
 *   type.
 *
 * Special values of the arguments:
 *   M == 0 or N == 0       nothing is done (returns DG_OK).
 *   K == 0 or alpha == 0   C = beta * C; A and B are not read.
 *   beta == 0              C is write-only: its old contents (NaN included)
 *                          are not read.
 *
 * Pointers, ownership, execution:
 *   A, B, C are device pointers on the device that `stream` belongs to, owned
 *   by the caller; the library keeps no reference after the call returns.
 *   `stream` is a hipStream_t (NULL = the default stream).  The call enqueues
 *   the work and returns without waiting for it (asynchronous, like any
 *   kernel launch); it allocates no memory.  Calls are thread-safe.
 *   C must not overlap A or B (not checked).
 *
 * Errors (return value):
 *   DG_OK (0)          enqueued (or nothing to do).
 *   -i                 argument i (1-based, in the order of dg_gemm's
 *                      parameters) is invalid: transA/transB not 0 or 1,
 *                      M/N/K negative or above 2^31-1, ld below its minimum,
 *                      NULL pointer with a non-empty extent, unknown dtype.
 *                      Nothing is enqueued.
 *   DG_ERR_UNSUPPORTED the forced kernel cannot run this problem.
 *   DG_ERR_SCRATCH     (dg_gemm_splitk_noalloc) more partials than the
 *                      library's scratch holds.
 *   DG_ERR_HIP         a HIP call failed; dg_last_hip_error() returns its
 *                      hipError_t (per calling thread).
 */
#ifndef DENSE_GEMM_H
#define DENSE_GEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enumerations are int-sized in both languages (C++ fixes the underlying
 * type, so that every int a caller passes is a value of the parameter's type
 * and the library's own range checks see it); the ABI passes them as int. */
#ifdef __cplusplus
#define DG_ENUM(name) enum name : int
#else
#define DG_ENUM(name) enum name
#endif

/* op(X): X as stored (N) or its transpose (T). */
typedef DG_ENUM(dg_op) { DG_OP_N = 0, DG_OP_T = 1 } dg_op_t;
/* Operand, accumulator and output types (see "Types" above). */
typedef DG_ENUM(dg_dtype) {
    DG_F32 = 0,          /* A, B, C fp32; fp32 accumulation            */
    DG_F16_F32ACC = 1,   /* A, B, C fp16; fp32 accumulation, fp16 out  */
    DG_BF16_F32ACC = 2,  /* A, B, C bf16; fp32 accumulation, bf16 out  */
    DG_F16_F32OUT = 3,   /* A, B fp16; fp32 accumulation, C fp32       */
    DG_BF16_F32OUT = 4   /* A, B bf16; fp32 accumulation, C fp32       */
} dg_dtype_t;
/* Epilogue activations of dg_gemm_ex. */
typedef DG_ENUM(dg_epilogue) { DG_EPI_NONE = 0, DG_EPI_RELU = 1, DG_EPI_GELU = 2 } dg_epilogue_t;
#undef DG_ENUM

#define DG_OK 0
#define DG_ERR_UNSUPPORTED (-100)
#define DG_ERR_SCRATCH (-101)
#define DG_ERR_HIP (-200)

/* Kernel choice for dg_gemm_with_kernel: DG_KERNEL_AUTO lets the library pick. */
#define DG_KERNEL_AUTO (-1)

/* C = alpha * op(A) * op(B) + beta * C  (see above). */
int dg_gemm(dg_op_t transA, dg_op_t transB, int64_t M, int64_t N, int64_t K, float alpha,
            const void *A, int64_t lda, const void *B, int64_t ldb, float beta, void *C,
            int64_t ldc, dg_dtype_t dtype, void *stream);

/* Same as dg_gemm, but runs kernel `kernel` (an index into the library's
 * kernel table, see dg_kernel_count / dg_kernel_name) instead of the one the
 * library would pick; DG_KERNEL_AUTO behaves as dg_gemm.  Returns
 * DG_ERR_UNSUPPORTED (nothing enqueued) when that kernel does not handle the
 * problem's dtype, transposes, alignment or row strides (the pipelined
 * kernels address a tile's operands with 32-bit byte offsets, so they need
 * 256 rows of the stored A and of the stored B to span less than 2^31
 * bytes).  For tests and measurement. */
int dg_gemm_with_kernel(dg_op_t transA, dg_op_t transB, int64_t M, int64_t N, int64_t K,
                        float alpha, const void *A, int64_t lda, const void *B, int64_t ldb, float beta,
                        void *C, int64_t ldc, dg_dtype_t dtype, void *stream, int kernel);

/* Extended form: a fused bias + activation epilogue and strided batches.
 *
 *   for b in 0 .. batch-1:
 *     C_b = act(alpha * op(A_b) * op(B_b) + beta * C_b + bias)
 *     with A_b = A + b*strideA, B_b = B + b*strideB, C_b = C + b*strideC
 *     (strides in elements).
 *
 * The epilogue is the fusion of "From a C loop to a GPU kernel", section
 * "Fusion": a per-output bias is added and an elementwise activation applied
 * while the tile is still on chip, and the result is written once.  In a
 * row-major C the outputs of one feature are a column, so bias[j] is added to
 * every element of column j:
 *   x = alpha*acc + beta*C_in + bias[j]   (in fp32, one rounding at the end)
 *   epilogue DG_EPI_NONE: x;  DG_EPI_RELU: max(x, 0) (NaN stays NaN);
 *   DG_EPI_GELU: x * Phi(x) = x/2 * (1 + erf(x / sqrt(2))), the exact-erf
 *   form, Phi the standard normal distribution function.
 * The batch is the per-head offset of "Metal GEMM Kernels for LoRA Training",
 * section 8 (Q, K, V head-major, one GEMM per head at a fixed offset): one
 * call runs every head, so the heads together fill the GPU.
 *
 * Arguments (1-based positions, for the -i error codes):
 *   1-8, 10-11, 13-15, 20-21: as dg_gemm's transA, transB, M, N, K, alpha,
 *       A, lda, B, ldb, beta, C, ldc, dtype, stream.
 *   9 strideA, 12 strideB: >= 0 (0 reuses one matrix for every batch).
 *   16 strideC: >= 0; with batch > 1 the outputs must not overlap:
 *       strideC >= (M-1)*ldc + N.
 *   17 batch: 0 .. 65535 (0: nothing is done).
 *   18 bias: NULL (no bias) or N elements of C's type, contiguous, aligned
 *       to its element size, shared by every batch; caller-owned device
 *       memory.
 *   19 epilogue: DG_EPI_NONE, DG_EPI_RELU or DG_EPI_GELU.
 * Special values as dg_gemm; with K == 0 or alpha == 0 the result is
 * act(beta*C + bias) and A and B are not read.  Pointer rules, asynchrony and
 * errors as dg_gemm (nothing enqueued on error).  No allocation. */
int dg_gemm_ex(dg_op_t transA, dg_op_t transB, int64_t M, int64_t N, int64_t K, float alpha,
               const void *A, int64_t lda, int64_t strideA, const void *B, int64_t ldb,
               int64_t strideB, float beta, void *C, int64_t ldc, int64_t strideC,
               int64_t batch, const void *bias, dg_epilogue_t epilogue, dg_dtype_t dtype,
               void *stream);

/* dg_gemm_ex with a forced kernel, as dg_gemm_with_kernel (argument 22). */
int dg_gemm_ex_with_kernel(dg_op_t transA, dg_op_t transB, int64_t M, int64_t N, int64_t K,
                           float alpha, const void *A, int64_t lda, int64_t strideA, const void *B,
                           int64_t ldb, int64_t strideB, float beta, void *C, int64_t ldc,
                           int64_t strideC, int64_t batch, const void *bias,
                           dg_epilogue_t epilogue, dg_dtype_t dtype, void *stream, int kernel);

/* Split-K form of dg_gemm, for outputs too small to give every compute unit a
 * tile (skinny and low-rank products): K is cut into `splits` ranges (each a
 * multiple of 64 long except the last), each range's products are summed
 * into fp32 partials in `workspace`, and a second kernel forms
 * C = alpha * (sum of the partials, in increasing range order) + beta * C with
 * one rounding to the output type.  This is the split-K remedy of "Metal
 * GEMM Kernels for LoRA Training on Apple Silicon", section 5 (fp32 partials,
 * then a reduction).
 *   splits      1: exactly dg_gemm (workspace unused); 0: the library's
 *               choice (dg_gemm_splitk_choose); n > 1: at most n ranges (the
 *               range length is rounded up to a multiple of 64, so fewer
 *               ranges may result).  Invalid (-16): below 0 or above 4096.
 *   workspace   device memory of at least dg_gemm_splitk_workspace_size(M,
 *               N, splits) bytes, 16-byte aligned, owned by the caller, not
 *               read or written outside that size; its contents on return
 *               are unspecified.  Invalid (-17): NULL or misaligned when
 *               splits != 1 and the output is not empty.  Too small for the
 *               ranges actually used: -18.  Two calls that share a workspace
 *               must be ordered on one stream.
 * Otherwise as dg_gemm (arguments 1-15, same errors, asynchronous). */
int dg_gemm_splitk(dg_op_t transA, dg_op_t transB, int64_t M, int64_t N, int64_t K, float alpha,
                   const void *A, int64_t lda, const void *B, int64_t ldb, float beta, void *C,
                   int64_t ldc, dg_dtype_t dtype, void *stream, int splits, void *workspace,
                   size_t workspace_bytes);

/* Bytes of the library's own split-K scratch on each GPU (see
 * dg_gemm_splitk_noalloc). */
#define DG_SCRATCH_BYTES (16 * 1024 * 1024)

/* dg_gemm_splitk without a workspace and without any allocation, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  The fp32 partials go to a
 * device array inside the library, DG_SCRATCH_BYTES (16 MiB) on each GPU,
 * which the GPU holds from the library's load until the process ends.  The
 * call uses the K ranges dg_gemm_splitk would use for the same `splits` (0:
 * the library's choice; 1: no split, the scratch is not touched), computes
 * the same result with the same kernels, and enqueues the same work.
 *   Arguments 1-16: as dg_gemm_splitk's first 16 (same errors, -16 for
 *   splits below 0 or above 4096).
 *   DG_ERR_SCRATCH: the partials, splits * M * N * 4 bytes for the ranges
 *   used, exceed DG_SCRATCH_BYTES; nothing is enqueued (call dg_gemm_splitk
 *   with a workspace, or fewer splits).
 *   DG_ERR_HIP: looking up the scratch's device address failed (first call
 *   on a device only).
 * Every call on one GPU shares that GPU's scratch, and a call leaves its
 * partials there: calls that may overlap on one GPU (on different streams,
 * or from several host threads without ordering) race on it and must be
 * ordered by the caller, for example on one stream.  No memory is cleared:
 * the GEMM kernel writes every partial before the reduction reads it.
 * Asynchronous, like dg_gemm; calls no allocating routine. */
int dg_gemm_splitk_noalloc(dg_op_t transA, dg_op_t transB, int64_t M, int64_t N, int64_t K,
                           float alpha, const void *A, int64_t lda, const void *B, int64_t ldb,
                           float beta, void *C, int64_t ldc, dg_dtype_t dtype, void *stream,
                           int splits);

/* The number of K ranges dg_gemm_splitk uses when called with splits = 0
 * (1 when splitting does not pay), or a negative status for invalid
 * arguments (host logic only). */
int dg_gemm_splitk_choose(dg_op_t transA, dg_op_t transB, int64_t M, int64_t N, int64_t K,
                          dg_dtype_t dtype);

/* Bytes of workspace dg_gemm_splitk needs for `splits` K ranges (0 when
 * splits <= 1 or the output is empty). */
size_t dg_gemm_splitk_workspace_size(int64_t M, int64_t N, int splits);

/* The kernel dg_gemm would run for these arguments (host logic only, no GPU
 * call), or a negative status as dg_gemm would return it. */
int dg_select_kernel(dg_op_t transA, dg_op_t transB, int64_t M, int64_t N, int64_t K, const void *A,
                     int64_t lda, const void *B, int64_t ldb, const void *C, int64_t ldc,
                     dg_dtype_t dtype);

/* Number of kernels in the table, and a static name for kernel i (NULL when
 * i is out of range).  Names read "<dtype>_<tiles>_<variant>". */
int dg_kernel_count(void);
const char *dg_kernel_name(int kernel);

/* Output tile (rows x cols of C per workgroup) of kernel i; -1 if out of range. */
int dg_kernel_tile_m(int kernel);
int dg_kernel_tile_n(int kernel);

/* Static text for a status code. */
const char *dg_status_string(int status);

/* hipError_t of the calling thread's last DG_ERR_HIP (0 if none). */
int dg_last_hip_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int dg_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DENSE_GEMM_H */
