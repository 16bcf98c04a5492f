// Host side of libdense_gemm_amd.so: argument validation, the kernel table,
// kernel selection and launch on the caller's stream.  The C ABI is declared
// in include/dense_gemm.h.
#include "../../include/dense_gemm.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "gemm_common.hpp"

// The split-K scratch of dg_gemm_splitk_noalloc (see scratch_for below).
static __device__ __align__(256) float scratch[DG_SCRATCH_BYTES / 4];

namespace dg {
launch_fn simple_launcher(int dtype, int ta, int tb);
launch_fn scale_launcher(int dtype);
launch_fn splitk_reduce_launcher(int dtype);
const launch_fn *f32_launchers(int config);
const launch_fn *f16_launchers(int config);
const launch_fn *f16_pipe_launchers(int config);
const launch_fn *f32_pipe_launchers(int config);
const launch_fn *bf16_pipe_launchers(int config);
const launch_fn *bf16_launchers(int config);
const launch_fn *f16_o32_launchers(int config);
const launch_fn *f16_o32_pipe_launchers(int config);
const launch_fn *bf16_o32_launchers(int config);
const launch_fn *bf16_o32_pipe_launchers(int config);
}  // namespace dg

namespace {

using dg::GemmParams;
using dg::launch_fn;

thread_local int g_last_hip_error = 0;

// One entry per compiled kernel family.
//   SIMPLE: generic fallback, any problem.
//   MFMA:   register-staged matrix-core kernels, any shape; 8 variants:
//           transA x transB x (16-byte vector loads or element loads).
//   PIPE:   direct-to-LDS pipelined kernels; 4 variants (transA x transB);
//           need 4-byte aligned rows of A and B, and the m/n-contiguous
//           operand's extent a multiple of 16 bytes.
//   PIPE_DW: pipelined kernels with 4-byte direct loads (fp32: 16-byte
//           ones for a k-contiguous operand in the _kw kernels); any fp32
//           layout (4-byte aligned A and B).
//   Both pipelined kinds address a tile's operands with 32-bit byte offsets.
// `dtype` is the operand type (DG_F32, DG_F16_F32ACC or DG_BF16_F32ACC); a
// 16-bit family serves both of its output types: `variants` writes C in the
// operand type, `variants32` the same kernels writing an fp32 C.
enum Kind { SIMPLE, MFMA, PIPE, PIPE_DW };
struct Family {
    const char *name;
    int dtype;
    int bm, bn;
    int group_m;
    Kind kind;
    const launch_fn *(*variants)(int);
    int config;
    const launch_fn *(*variants32)(int);
};

const Family kFamilies[] = {
    {"f32_64x64_simple", DG_F32, 64, 64, 1, SIMPLE, nullptr, 0},
    {"f16_64x64_simple", DG_F16_F32ACC, 64, 64, 1, SIMPLE, nullptr, 0},
    {"f32_256x128_mfma32x32x2", DG_F32, 256, 128, 8, MFMA, dg::f32_launchers, 0},
    {"f32_128x128_mfma32x32x2", DG_F32, 128, 128, 8, MFMA, dg::f32_launchers, 1},
    {"f16_128x128_mfma32x32x16", DG_F16_F32ACC, 128, 128, 4, MFMA, dg::f16_launchers, 0, dg::f16_o32_launchers},
    {"f16_256x128_mfma32x32x16", DG_F16_F32ACC, 256, 128, 4, MFMA, dg::f16_launchers, 1, dg::f16_o32_launchers},
    {"f16_128x128_pipe4_ksplit2_mfma32x32x16", DG_F16_F32ACC, 128, 128, 4, PIPE, dg::f16_pipe_launchers, 0, dg::f16_o32_pipe_launchers},
    {"f16_256x128_pipe2_w8_mfma32x32x16", DG_F16_F32ACC, 256, 128, 4, PIPE, dg::f16_pipe_launchers, 1, dg::f16_o32_pipe_launchers},
    {"f16_128x128_pipe2_ksplit2_mfma32x32x16", DG_F16_F32ACC, 128, 128, 4, PIPE, dg::f16_pipe_launchers, 2, dg::f16_o32_pipe_launchers},
    {"f32_256x128_pipe3_mfma32x32x2", DG_F32, 256, 128, 8, PIPE, dg::f32_pipe_launchers, 0},
    {"f32_256x256_pipe4_w8_mfma32x32x2", DG_F32, 256, 256, 4, PIPE, dg::f32_pipe_launchers, 1},
    {"f32_128x128_pipe4_mfma32x32x2", DG_F32, 128, 128, 8, PIPE, dg::f32_pipe_launchers, 2},
    {"bf16_64x64_simple", DG_BF16_F32ACC, 64, 64, 1, SIMPLE, nullptr, 0},
    {"bf16_128x128_pipe4_ksplit2_mfma32x32x16", DG_BF16_F32ACC, 128, 128, 4, PIPE, dg::bf16_pipe_launchers, 0, dg::bf16_o32_pipe_launchers},
    {"bf16_256x128_pipe2_w8_mfma32x32x16", DG_BF16_F32ACC, 256, 128, 4, PIPE, dg::bf16_pipe_launchers, 1, dg::bf16_o32_pipe_launchers},
    {"bf16_128x128_pipe2_ksplit2_mfma32x32x16", DG_BF16_F32ACC, 128, 128, 4, PIPE, dg::bf16_pipe_launchers, 2, dg::bf16_o32_pipe_launchers},
    {"f16_64x64_pipe4_ksplit2_mfma32x32x16", DG_F16_F32ACC, 64, 64, 4, PIPE, dg::f16_pipe_launchers, 3, dg::f16_o32_pipe_launchers},
    {"f16_128x32_pipe4_mfma32x32x16", DG_F16_F32ACC, 128, 32, 4, PIPE, dg::f16_pipe_launchers, 4, dg::f16_o32_pipe_launchers},
    {"f16_32x128_pipe4_mfma32x32x16", DG_F16_F32ACC, 32, 128, 4, PIPE, dg::f16_pipe_launchers, 5, dg::f16_o32_pipe_launchers},
    {"bf16_64x64_pipe4_ksplit2_mfma32x32x16", DG_BF16_F32ACC, 64, 64, 4, PIPE, dg::bf16_pipe_launchers, 3, dg::bf16_o32_pipe_launchers},
    {"bf16_128x32_pipe4_mfma32x32x16", DG_BF16_F32ACC, 128, 32, 4, PIPE, dg::bf16_pipe_launchers, 4, dg::bf16_o32_pipe_launchers},
    {"bf16_32x128_pipe4_mfma32x32x16", DG_BF16_F32ACC, 32, 128, 4, PIPE, dg::bf16_pipe_launchers, 5, dg::bf16_o32_pipe_launchers},
    {"f16_256x256_pipe2_w8_mfma32x32x16", DG_F16_F32ACC, 256, 256, 4, PIPE, dg::f16_pipe_launchers, 6, dg::f16_o32_pipe_launchers},
    {"bf16_256x256_pipe2_w8_mfma32x32x16", DG_BF16_F32ACC, 256, 256, 4, PIPE, dg::bf16_pipe_launchers, 6, dg::bf16_o32_pipe_launchers},
    {"f32_256x128_pipe3_dw_mfma32x32x2", DG_F32, 256, 128, 8, PIPE_DW, dg::f32_pipe_launchers, 3},
    {"f32_128x128_pipe4_dw_mfma32x32x2", DG_F32, 128, 128, 8, PIPE_DW, dg::f32_pipe_launchers, 4},
    {"f16_128x128_pipe4_ksplit2_dw_mfma32x32x16", DG_F16_F32ACC, 128, 128, 4, PIPE_DW, dg::f16_pipe_launchers, 7, dg::f16_o32_pipe_launchers},
    {"f16_64x64_pipe4_ksplit2_dw_mfma32x32x16", DG_F16_F32ACC, 64, 64, 4, PIPE_DW, dg::f16_pipe_launchers, 8, dg::f16_o32_pipe_launchers},
    {"bf16_128x128_pipe4_ksplit2_dw_mfma32x32x16", DG_BF16_F32ACC, 128, 128, 4, PIPE_DW, dg::bf16_pipe_launchers, 7, dg::bf16_o32_pipe_launchers},
    {"bf16_64x64_pipe4_ksplit2_dw_mfma32x32x16", DG_BF16_F32ACC, 64, 64, 4, PIPE_DW, dg::bf16_pipe_launchers, 8, dg::bf16_o32_pipe_launchers},
    {"bf16_128x128_mfma32x32x16", DG_BF16_F32ACC, 128, 128, 4, MFMA, dg::bf16_launchers, 0, dg::bf16_o32_launchers},
    {"bf16_256x128_mfma32x32x16", DG_BF16_F32ACC, 256, 128, 4, MFMA, dg::bf16_launchers, 1, dg::bf16_o32_launchers},
    {"f32_128x64_pipe4_mfma32x32x2", DG_F32, 128, 64, 8, PIPE, dg::f32_pipe_launchers, 5},
    {"f32_64x64_pipe4_mfma32x32x2", DG_F32, 64, 64, 8, PIPE, dg::f32_pipe_launchers, 6},
    {"f32_128x64_pipe4_dw_mfma32x32x2", DG_F32, 128, 64, 8, PIPE_DW, dg::f32_pipe_launchers, 7},
    {"f32_64x64_pipe4_dw_mfma32x32x2", DG_F32, 64, 64, 8, PIPE_DW, dg::f32_pipe_launchers, 8},
    {"f32_64x64_pipe3_k32_mfma32x32x2", DG_F32, 64, 64, 8, PIPE, dg::f32_pipe_launchers, 9},
    {"f32_32x32_pipe3_k32_ksplit4_mfma32x32x2", DG_F32, 32, 32, 8, PIPE, dg::f32_pipe_launchers, 10},
    {"f32_32x32_pipe4_k32_ksplit4_mfma32x32x2", DG_F32, 32, 32, 8, PIPE, dg::f32_pipe_launchers, 11},
    {"f32_64x64_pipe4_kw_mfma32x32x2", DG_F32, 64, 64, 8, PIPE_DW, dg::f32_pipe_launchers, 12},
    {"f32_64x64_pipe3_k32_kw_mfma32x32x2", DG_F32, 64, 64, 8, PIPE_DW, dg::f32_pipe_launchers, 13},
};
constexpr int kNumKernels = sizeof(kFamilies) / sizeof(kFamilies[0]);
enum {
    K_F32_SIMPLE = 0, K_F16_SIMPLE = 1, K_F32_256 = 2, K_F32_128 = 3, K_F16_128 = 4, K_F16_256 = 5,
    K_F16_PIPE_128 = 6, K_F16_PIPE_256 = 7, K_F16_PIPE_128_2 = 8, K_F32_PIPE_256x128 = 9,
    K_F32_PIPE_256x256 = 10, K_F32_PIPE_128 = 11, K_BF16_SIMPLE = 12, K_BF16_PIPE_128 = 13,
    K_BF16_PIPE_256 = 14, K_BF16_PIPE_128_2 = 15, K_F16_PIPE_64 = 16, K_F16_PIPE_128x32 = 17,
    K_F16_PIPE_32x128 = 18, K_BF16_PIPE_64 = 19, K_BF16_PIPE_128x32 = 20, K_BF16_PIPE_32x128 = 21,
    K_F16_PIPE_256x256 = 22, K_BF16_PIPE_256x256 = 23, K_F32_PIPE_256x128_DW = 24,
    K_F32_PIPE_128_DW = 25, K_F16_PIPE_128_DW = 26, K_F16_PIPE_64_DW = 27, K_BF16_PIPE_128_DW = 28,
    K_BF16_PIPE_64_DW = 29, K_BF16_128 = 30, K_BF16_256 = 31, K_F32_PIPE_128x64 = 32,
    K_F32_PIPE_64 = 33, K_F32_PIPE_128x64_DW = 34, K_F32_PIPE_64_DW = 35, K_F32_PIPE_64_K32 = 36,
    K_F32_PIPE_32_KG4 = 37, K_F32_PIPE_32_KG4_S4 = 38, K_F32_PIPE_64_KW = 39, K_F32_PIPE_64_K32_KW = 40
};

constexpr int64_t kMaxBatch = 65535;   // a grid dimension

// The strided-batch and epilogue arguments of dg_gemm_ex (defaults: one
// matrix, no bias, no activation).
struct Ext {
    int64_t sA = 0, sB = 0, sC = 0;
    int64_t batch = 1;
    const void *bias = nullptr;
    int act = DG_EPI_NONE;
};

bool is_dtype(int dtype)
{
    return dtype == DG_F32 || dtype == DG_F16_F32ACC || dtype == DG_BF16_F32ACC ||
           dtype == DG_F16_F32OUT || dtype == DG_BF16_F32OUT;
}

// The operand type of a dtype (the type the kernel table is keyed by).
int op_dtype(int dtype)
{
    return dtype == DG_F16_F32OUT ? DG_F16_F32ACC : dtype == DG_BF16_F32OUT ? DG_BF16_F32ACC : dtype;
}

// Bytes of one element of A and B.
int64_t elem_bytes(int dtype) { return op_dtype(dtype) == DG_F32 ? 4 : 2; }

// Bytes of one element of C (and of the bias).
int64_t c_bytes(int dtype) { return (dtype == DG_F16_F32ACC || dtype == DG_BF16_F32ACC) ? 2 : 4; }

constexpr int64_t kMaxDim = 0x7fffffff;

int64_t max1(int64_t x) { return x > 1 ? x : 1; }

// Argument checks in parameter order; returns 0 or -(1-based index).
// check_ptrs = false skips the NULL checks (kernel selection only looks at
// shapes, strides and alignment).
int validate(int ta, int tb, int64_t M, int64_t N, int64_t K, float alpha, const void *A,
             int64_t lda, const void *B, int64_t ldb, const void *C, int64_t ldc, int dtype,
             bool check_ptrs = true)
{
    if (ta != DG_OP_N && ta != DG_OP_T) return -1;
    if (tb != DG_OP_N && tb != DG_OP_T) return -2;
    if (M < 0 || M > kMaxDim) return -3;
    if (N < 0 || N > kMaxDim) return -4;
    if (K < 0 || K > kMaxDim) return -5;
    const bool reads_ab = check_ptrs && M > 0 && N > 0 && K > 0 && alpha != 0.f;
    if (reads_ab && A == nullptr) return -7;
    if (lda < max1(ta == DG_OP_T ? M : K)) return -8;
    if (reads_ab && B == nullptr) return -9;
    if (ldb < max1(tb == DG_OP_T ? K : N)) return -10;
    if (check_ptrs && M > 0 && N > 0 && C == nullptr) return -12;
    if (ldc < max1(N)) return -13;
    if (!is_dtype(dtype)) return -14;
    return 0;
}

// The extended arguments (batch strides, batch count, bias, activation) in
// dg_gemm_ex's parameter order; returns 0 or -(1-based index there).
int validate_ext(int64_t M, int64_t N, int64_t ldc, const Ext &x, int dtype)
{
    if (x.sA < 0) return -9;
    if (x.sB < 0) return -12;
    // batches of C must not overlap: batch b+1 starts past the last element of batch b
    if (x.sC < 0 || (x.batch > 1 && M > 0 && N > 0 && x.sC < (M - 1) * ldc + N)) return -16;
    if (x.batch < 0 || x.batch > kMaxBatch) return -17;
    if (x.bias && ((uintptr_t)x.bias % (uintptr_t)c_bytes(dtype)) != 0) return -18;
    if (x.act != DG_EPI_NONE && x.act != DG_EPI_RELU && x.act != DG_EPI_GELU) return -19;
    return 0;
}

// dg_gemm's argument position -> dg_gemm_ex's (the extended form inserts the
// batch strides after lda, ldb and ldc, and batch, bias, epilogue before dtype).
int ex_position(int rc)
{
    switch (rc) {
    case -9: return -10;    // B
    case -10: return -11;   // ldb
    case -11: return -13;   // beta
    case -12: return -14;   // C
    case -13: return -15;   // ldc
    case -14: return -20;   // dtype
    default: return rc;     // transA .. lda keep their positions
    }
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

// Every row start of C (in every batch) on a 4-byte boundary: the epilogue
// then reads and writes C in 16-byte pieces (whole multiples of 16 bytes from
// a row start, so each access is at least 4-byte aligned: the same alignment
// the k-contiguous operands' 16-byte direct loads run at), else element by
// element.  Always so for an fp32 C; a 16-bit C needs an even ldc.
bool c_rows_vec(const void *C, int64_t ldc, int dtype, const Ext &x)
{
    const int64_t cb = c_bytes(dtype);
    return ((uintptr_t)C & 3) == 0 && (ldc * cb) % 4 == 0 && (x.batch <= 1 || (x.sC * cb) % 4 == 0);
}

// 16-byte vector loads need every row start of A and B on a 16-byte boundary
// (in every batch: the batch strides are whole 16-byte pieces too).
bool vec_ok(const void *A, int64_t lda, const void *B, int64_t ldb, int dtype, const Ext &x)
{
    const int64_t v = 16 / elem_bytes(dtype);
    return aligned16(A) && aligned16(B) && lda % v == 0 && ldb % v == 0 &&
           (x.batch <= 1 || (x.sA % v == 0 && x.sB % v == 0));
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The direct loads address a tile panel with 32-bit byte offsets, at most
// 256 rows of the stored matrix from the panel's origin.
bool offsets_fit(int64_t lda, int64_t ldb, int dtype)
{
    const int64_t lim = (int64_t)1 << 31;
    return 256 * lda * elem_bytes(dtype) < lim && 256 * ldb * elem_bytes(dtype) < lim;
}

// Preconditions of the pipelined kernels (see Family): 4-byte aligned rows
// of A and B, and the m/n-contiguous operand's extent a whole number of
// 16-byte pieces.
// The 16-byte direct loads of a tile sit at whole multiples of 16 bytes from
// a row start, so they need every row start (in every batch) 4-byte aligned
// only, as the k-contiguous operands' 16-byte loads at padded rows do.
bool rows4_ok(const void *A, int64_t lda, const void *B, int64_t ldb, int dtype, const Ext &x)
{
    const int64_t eb = elem_bytes(dtype);
    return ((uintptr_t)A & 3) == 0 && ((uintptr_t)B & 3) == 0 && (lda * eb) % 4 == 0 &&
           (ldb * eb) % 4 == 0 && (x.batch <= 1 || ((x.sA * eb) % 4 == 0 && (x.sB * eb) % 4 == 0));
}

bool pipe_ok(int ta, int tb, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
             const void *B, int64_t ldb, int dtype, const Ext &x)
{
    const int64_t v = 16 / elem_bytes(dtype);
    (void)K;
    return offsets_fit(lda, ldb, dtype) && rows4_ok(A, lda, B, ldb, dtype, x) && (!ta || M % v == 0) &&
           (tb || N % v == 0);
}

// Preconditions of the pipelined kernels with 4-byte loads: 4-byte aligned
// rows of A and B; for 16-bit operands (a load takes an element pair) also
// even row strides and batch strides, and an even m/n-contiguous extent, so
// that no pair reaches past a row's last element.
bool pipe_dw_ok(int ta, int tb, int64_t M, int64_t N, const void *A, int64_t lda, const void *B,
                int64_t ldb, int dtype, const Ext &x)
{
    if (((uintptr_t)A & 3) != 0 || ((uintptr_t)B & 3) != 0 || !offsets_fit(lda, ldb, dtype)) return false;
    if (dtype == DG_F32) return true;
    return lda % 2 == 0 && ldb % 2 == 0 && (x.batch <= 1 || (x.sA % 2 == 0 && x.sB % 2 == 0)) &&
           (!ta || M % 2 == 0) && (tb || N % 2 == 0);
}

// The 4-byte-load counterpart of a 16-byte-load 16-bit kernel: the 64x64
// tile for the narrow ones, else the 128x128 tile (the larger tiles with
// 4-byte loads would spill their per-lane offsets).
int dw_kernel(int k, bool bf)
{
    switch (k) {
    case K_F16_PIPE_64: case K_F16_PIPE_128x32: case K_F16_PIPE_32x128:
    case K_BF16_PIPE_64: case K_BF16_PIPE_128x32: case K_BF16_PIPE_32x128:
        return bf ? K_BF16_PIPE_64_DW : K_F16_PIPE_64_DW;
    default:
        return bf ? K_BF16_PIPE_128_DW : K_F16_PIPE_128_DW;
    }
}

// Kernel choice by dtype, preconditions and output tile count.  Larger tiles
// re-read less of A and B; smaller tiles fill more of the 256 compute units.
int choose(int ta, int tb, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
           const void *B, int64_t ldb, int dtype, const Ext &x = Ext(), bool c_vec = true)
{
    // the output type does not change the choice: the kernels are the same
    dtype = op_dtype(dtype);
    // a batch multiplies the workgroups: count the tiles of all batches
    const int64_t nb = x.batch > 1 ? x.batch : 1;
    const int64_t big = ceil_div(M, 256) * ceil_div(N, 128) * nb;
    const int64_t small = ceil_div(M, 128) * ceil_div(N, 128) * nb;
    const bool pipe = pipe_ok(ta, tb, M, N, K, A, lda, B, ldb, dtype, x);
    if (dtype == DG_F32) {
        // The tile by its cost in rounds: a CU runs its share of the tiles in
        // about ceil(tiles / 256) tile-times, whether one or two of them are
        // resident, and a tile's time relative to a 128x128 one is 1.933
        // (256x128), 0.51 (128x64) and 0.2636 (64x64).  Measured at 4096^3,
        // the model then matched the fastest tile at 6144^3, 3584^3, 2560^3,
        // 4096x4224x4096, 3072x4096x4096, 5120x4096x2048, 6144^2x2048,
        // 2304x2048x2048, 2048x3072x2048, 8192^2x2048, 4096^2x1024 and
        // 1024x16384x4096 (within 2-3% of its prediction).  256x128 is
        // considered only when its tiles fill whole rounds of two per CU: with
        // a partly filled last round it ran 20-27% slower than predicted
        // (6144^3, 5120x4096x2048).  Small tiles win where the larger ones end
        // in a partly filled round: 4095x4097x1031 (the 4097th column adds a
        // whole tile column) 302-345 us against 410-498 on 128x128, 3584^3
        // 729 against 822 on 256x128.  At most one 128x128 tile per CU: the
        // 64x64 tile (two or more workgroups per CU), measured 8192x256x8192
        // 291-295 against 510-521 us on 128x128 (all four transpose pairs),
        // 512^3 15 against 40, 1024^3 28 against 73, 512^2x8192 176 against
        // 515, 3072x1024x2048 106 against 139, 2048^3 134 against 139.
        const int64_t t12864 = ceil_div(M, 128) * ceil_div(N, 64) * nb;
        const int64_t t64 = ceil_div(M, 64) * ceil_div(N, 64) * nb;
        int pk;                                    // 0: 256x128, 1: 128x128, 2: 128x64, 3: 64x64
        const double cost[4] = {(big % 512 == 0) ? ceil_div(big, 256) * 1.933 : 1e30,
                                (double)ceil_div(small, 256),
                                ceil_div(t12864, 256) * 0.51, ceil_div(t64, 256) * 0.2636};
        if (small <= 256) {
            pk = 3;
        } else {
            pk = 0;
            for (int c = 1; c < 4; ++c)
                if (cost[c] < cost[pk]) pk = c;
        }
        static const int pipe16[4] = {K_F32_PIPE_256x128, K_F32_PIPE_128, K_F32_PIPE_128x64, K_F32_PIPE_64};
        static const int pipe4[4] = {K_F32_PIPE_256x128_DW, K_F32_PIPE_128_DW, K_F32_PIPE_128x64_DW, K_F32_PIPE_64_DW};
        if (pipe) {
            // The 64x64 tile with 32-deep slabs (each k-contiguous row of a
            // stage one whole 128-byte line) in three stages, 48 KB of LDS, so
            // three workgroups per CU.  Against the 16-deep four-stage kernel
            // (32 KB, four resident per CU), one machine: 512^3 7-9% faster,
            // 1024^3 7-9%, 1024^2x4096 and 512^2x8192 8-10%, 8192x256x8192
            // (ld + 8) 3-6% for nn, nt and tt (tn even), 2304x2048^2 5-10%,
            // 3072^3 4-5%.  Grids of 769 to 1024 tiles fill one round of four
            // per CU but need two of three: there the 16-deep kernel stays
            // (2048^3 and 2048^2x1024 nt, tn, tt 3-19% slower on the 32-deep
            // one, 1792^2x2048 2-4%).
            //
            // Fewer 64x64 tiles than CUs: the 32x32 tile with four K groups,
            // one wave per SIMD for each tile, so four times the tiles and
            // every SIMD of their CUs at work.  Against the 64x64 32-deep
            // kernel, one machine: 512^3 5.4-6.1 against 11.8-12.4 us (all
            // four transpose pairs), 256^3 4.5 against 8.1, 768^3 14.2
            // against 17.2, 512^2x2048 15.7 against 37.6, 512^2x8192 60
            // against 138; even at 256 tiles (1024^3 21.7 against 21.8,
            // 2048x512x512 13.1 against 13.3), 6% slower at 1024^2x4096.
            // From K = 512 the four-stage kernel, whose loop reads each
            // slab's fragments one step ahead (nn, nt, tt): 512^3 nn/nt/tn/tt
            // 5.93/5.58/6.13/6.02 us against 6.23/5.52/6.02/6.20 with three
            // stages, 768^3 nn 13.4 against 14.2, 512^2x1024 8.1/7.5/8.9/8.2
            // against 9.2/7.7/8.9/9.1, 512^2x8192 41.3/37.8/50.8/41.9 against
            // 59.8/48.9/62.7/59.8; below K = 512 three stages (1-5% faster at
            // K = 128 and 256).
            if (pk == 3 && t64 < 256) return K >= 512 ? K_F32_PIPE_32_KG4_S4 : K_F32_PIPE_32_KG4;
            if (pk == 3 && (t64 <= 768 || t64 > 1024)) return K_F32_PIPE_64_K32;
            return pipe16[pk];
        }
        // rows not 16-byte aligned: the same tiles with 4-byte direct loads
        // (the 32-deep slab measured 38% slower with them: 4095x4097x1031).
        // On the 64x64 tile a k-contiguous operand takes 16-byte loads all
        // the same (its pieces never cross the end of a row), one machine,
        // 4095x4097x1031 with ld + 8: nn and tt 320.5 / 320.7 us against
        // 330.4 / 331.0 (16-deep), nt 307.4 against 345.9 (32-deep, both
        // operands k-contiguous); 2047x2049x2051 3-14% faster.  tn has no
        // k-contiguous operand and keeps the 4-byte kernel.
        if (pipe_dw_ok(ta, tb, M, N, A, lda, B, ldb, dtype, x)) {
            if (pk == 3 && !(ta && !tb)) return (!ta && tb) ? K_F32_PIPE_64_K32_KW : K_F32_PIPE_64_KW;
            return pipe4[pk];
        }
        return big >= 384 ? K_F32_256 : K_F32_128;
    }
    // 16-bit operands: the tile is picked by how many CUs its tiles fill
    const bool bf = dtype == DG_BF16_F32ACC;
    auto pick = [&]() -> int {
        // narrow outputs take tiles that match them instead of padding a
        // 128-wide tile: N or M of 32 (low-rank products), 64 (attention's
        // per-head products with d_head = 64)
        if (N <= 32) return bf ? K_BF16_PIPE_128x32 : K_F16_PIPE_128x32;
        if (M <= 32) return bf ? K_BF16_PIPE_32x128 : K_F16_PIPE_32x128;
        if (N <= 64 || M <= 64) return bf ? K_BF16_PIPE_64 : K_F16_PIPE_64;
        // a single K slab: writing C dominates, the large tile fills the GPU
        // once there is one per CU (attention's Q K^T, measured)
        if (K <= 64 && big >= 256) return bf ? K_BF16_PIPE_256 : K_F16_PIPE_256;
        // More than half the CUs with a 256x128 tile: the tile by its time in
        // rounds.  Each of these kernels runs one workgroup per CU, so the
        // tiles go in rounds of 256, and a partly filled last round costs
        // about 0.82 of a full one.  A round takes a fixed part (launch,
        // prologue, K-group sum, epilogue) and a part per unit of K: 128x128
        // 4.67 us + 7.52 ns per k, 256x128 7.07 us + 14.78 ns, 256x256 16.29
        // us + 21.44 ns, a least-squares fit to the times of the three tiles
        // at 39 shapes (1536-8448 x 1024-8192 x 512-8192, all three transpose
        // pairs; 5% rms error).  Over those 111 cases the tile chosen was
        // within 3% of the fastest of the four in 108, and 5-9% slower in
        // three (7168^2x1024 nn, nt; 4096^2x512 nn).  Examples: 4096^3, 6144^3
        // and 8448x4096x2048 take 256x256, 2048x4096x4096, 2304x2048^2 and
        // 4608^2x2048 take 256x128, 4608x4096x4096, 4224^3 and
        // 5120x4096x2048 take 128x128 (a few 256x256 tiles past a round).
        // The two-workgroup 128x128 kernel measured slower than the
        // one-workgroup one at every such shape and is not chosen.
        // C rows not 4-byte aligned (odd ldc): C goes through the epilogue
        // element by element, 2-3x slower on every tile, and the one-round
        // 256x256 and 256x128 grids run it on all CUs at once at the end.
        // fp16 C with ldc = N + 1, beta -0.5, nn/nt/tn, one machine: the 128x128 tile
        // 3-43% faster than the model's tile (4096^2x1032, 4096x8192x1032,
        // 2048x4096x520, 4096^3, 8192^2x1032; 256x256 2% ahead at 8192^2 nt).
        if (big > 128 && !c_vec) return bf ? K_BF16_PIPE_128 : K_F16_PIPE_128;
        if (big > 128) {
            auto rounds = [](int64_t t) { return (double)(t / 256) + (t % 256 ? 0.82 : 0.0); };
            const double k = (double)K;
            const int64_t t256 = ceil_div(M, 256) * ceil_div(N, 256) * nb;
            const double c256x256 = rounds(t256) * (16.29 + 0.02144 * k);
            const double c256x128 = rounds(big) * (7.07 + 0.01478 * k);
            const double c128 = rounds(small) * (4.67 + 0.00752 * k);
            if (c128 < c256x128 && c128 < c256x256) return bf ? K_BF16_PIPE_128 : K_F16_PIPE_128;
            if (c256x128 < c256x256) return bf ? K_BF16_PIPE_256 : K_F16_PIPE_256;
            return bf ? K_BF16_PIPE_256x256 : K_F16_PIPE_256x256;
        }
        // fewer 128x128 tiles than half the CUs and K too short to split:
        // smaller tiles (the LoRA K = 32 products, measured)
        if (small < 128 && K < 1024) return bf ? K_BF16_PIPE_64 : K_F16_PIPE_64;
        // at most half the CUs with a 128x128 tile while 64x64 tiles cover
        // them all: the 64x64 kernel without a K split.  Measured at 512x2048,
        // 1024x1024, 768x1536 and 512x4096 for K from 1024 to 8192: 7.7 us
        // against 24.5 for the 128x128 tile split four ways at K = 1024 (the
        // fp32 partials outweigh the output), 26 against 31 at K = 5632 (the
        // LoRA down and dH products).  From K = 16384 the split 128x128 tile
        // wins again (56 against 66 us).
        const int64_t t64 = ceil_div(M, 64) * ceil_div(N, 64) * nb;
        if (small <= 128 && t64 >= 256 && K <= 8192) return bf ? K_BF16_PIPE_64 : K_F16_PIPE_64;
        return bf ? K_BF16_PIPE_128 : K_F16_PIPE_128;
    };
    if (pipe) return pick();
    // rows 4-byte but not 16-byte aligned: the same tiles with 4-byte loads
    if (pipe_dw_ok(ta, tb, M, N, A, lda, B, ldb, dtype, x)) return dw_kernel(pick(), bf);
    if (bf) return big >= 512 ? K_BF16_256 : K_BF16_128;
    return big >= 512 ? K_F16_256 : K_F16_128;
}

bool supports(int kernel, int ta, int tb, int64_t M, int64_t N, int64_t K, const void *A,
              int64_t lda, const void *B, int64_t ldb, int dtype, const Ext &x)
{
    if (kernel < 0 || kernel >= kNumKernels) return false;
    const Family &f = kFamilies[kernel];
    if (f.dtype != op_dtype(dtype)) return false;
    if (f.kind == SIMPLE) return ceil_div(M, 64) <= 65535;
    if (f.kind == PIPE && !pipe_ok(ta, tb, M, N, K, A, lda, B, ldb, dtype, x)) return false;
    if (f.kind == PIPE_DW && !pipe_dw_ok(ta, tb, M, N, A, lda, B, ldb, dtype, x)) return false;
    return ceil_div(M, f.bm) * ceil_div(N, f.bn) <= 0x7fffffff;
}

// Number of K splits for a problem whose output has `tiles` tiles: enough
// workgroups to cover the 256 compute units, at least 4 K slabs of 64 per
// split; no split once half the compute units have a tile, nor for K below
// 1024, where the reduction's launch costs more than the split saves
// (measured on the LoRA step's K = 512 products).
int splits_for(int64_t tiles, int64_t K)
{
    if (tiles >= 128 || K < 1024) return 1;
    const int64_t want = ceil_div(256, tiles);
    const int64_t slabs = ceil_div(K, 64);
    int64_t s = slabs / 4;
    if (s > want) s = want;
    if (s < 1) s = 1;
    return (int)s;
}

// The K ranges a call runs with on kernel family f: `splits` (0: the
// library's choice for f's tile count) turned into ranges whose length is a
// multiple of 64 (every kernel's K slab divides it).  1 when the generic
// kernel runs (it has no split mode) or the ranges collapse into one;
// *k_chunk receives the range length (0 without a split).
int resolve_splits(const Family &f, int64_t M, int64_t N, int64_t K, int splits, int32_t *k_chunk)
{
    *k_chunk = 0;
    if (f.kind == SIMPLE || K == 0) return 1;
    if (splits == 0) splits = splits_for(ceil_div(M, f.bm) * ceil_div(N, f.bn), K);
    if (splits <= 1) return 1;
    const int64_t chunk = ceil_div(ceil_div(K, splits), 64) * 64;
    const int64_t n = ceil_div(K, chunk);
    if (n <= 1) return 1;
    *k_chunk = (int32_t)chunk;
    return (int)n;
}

int run(int ta, int tb, int64_t M, int64_t N, int64_t K, float alpha, const void *A, int64_t lda,
        const void *B, int64_t ldb, float beta, void *C, int64_t ldc, int dtype, void *stream,
        int kernel, int splits = 1, void *ws = nullptr, size_t ws_bytes = 0, const Ext &x = Ext())
{
    int rc = validate(ta, tb, M, N, K, alpha, A, lda, B, ldb, C, ldc, dtype, x.batch > 0);
    if (rc) return rc;
    if (M == 0 || N == 0 || x.batch == 0) return DG_OK;
    if (kernel != DG_KERNEL_AUTO && (kernel < 0 || kernel >= kNumKernels))
        return DG_ERR_UNSUPPORTED;

    GemmParams p;
    p.A = A;
    p.B = B;
    p.C = C;
    p.lda = lda;
    p.ldb = ldb;
    p.ldc = ldc;
    p.M = (int32_t)M;
    p.N = (int32_t)N;
    p.K = (int32_t)K;
    p.alpha = alpha;
    p.beta = beta;
    p.tiles_m = p.tiles_n = 0;
    p.group_m = 1;
    p.c_vec = c_rows_vec(C, ldc, dtype, x);
    p.splits = 1;
    p.k_chunk = 0;
    p.ws = nullptr;
    p.bias = x.bias;
    p.act = x.act;
    p.strideA = x.sA;
    p.strideB = x.sB;
    p.strideC = x.sC;
    p.batch = (int32_t)x.batch;
    hipStream_t s = (hipStream_t)stream;
    const int di = dtype;   // the generic launcher tables are indexed by dtype
    const bool out32 = dtype == DG_F16_F32OUT || dtype == DG_BF16_F32OUT;

    hipError_t err;
    if (K == 0 || alpha == 0.f) {
        err = dg::scale_launcher(di)(p, s);
    } else {
        if (kernel == DG_KERNEL_AUTO) kernel = choose(ta, tb, M, N, K, A, lda, B, ldb, dtype, x, p.c_vec);
        if (!supports(kernel, ta, tb, M, N, K, A, lda, B, ldb, dtype, x)) return DG_ERR_UNSUPPORTED;
        const Family &f = kFamilies[kernel];
        if (f.kind == SIMPLE) {
            err = dg::simple_launcher(di, ta, tb)(p, s);
        } else {
            p.tiles_m = (int32_t)ceil_div(M, f.bm);
            p.tiles_n = (int32_t)ceil_div(N, f.bn);
            p.group_m = f.group_m;
            p.splits = resolve_splits(f, M, N, K, splits, &p.k_chunk);
            if (p.splits > 1) {
                if ((size_t)p.splits * (size_t)M * (size_t)N * 4 > ws_bytes) return -18;
                p.ws = (float *)ws;
            }
            const int vi = (f.kind == PIPE || f.kind == PIPE_DW || vec_ok(A, lda, B, ldb, dtype, x)) ? 0 : 4;
            err = (out32 ? f.variants32 : f.variants)(f.config)[vi + ta * 2 + tb](p, s);
            if (err == hipSuccess && p.splits > 1) err = dg::splitk_reduce_launcher(di)(p, s);
        }
    }
    if (err != hipSuccess) {
        g_last_hip_error = (int)err;
        return DG_ERR_HIP;
    }
    return DG_OK;
}

// ---- scratch memory of dg_gemm_splitk_noalloc ---------------------------------
// The split-K partials of the allocation-free entry point live in this
// device array, one copy per GPU (each device that loads the library's code
// object gets its own), held until the process ends.  Host code never uses
// the array's name as an address: its device address is looked up once per
// device with hipGetSymbolAddress and kept in g_scratch.
constexpr int kMaxDevices = 64;

std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices] = {};

// The device address of `scratch` on the device `stream` belongs to (the
// current device for the NULL stream), looked up on first use with that
// device current.  Returns 0 or DG_ERR_HIP.
int scratch_for(void *stream, void **out)
{
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice((hipStream_t)stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return DG_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        g_last_hip_error = (int)hipErrorInvalidDevice;
        return DG_ERR_HIP;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch[dev] == nullptr) {
        int cur = 0;
        e = hipGetDevice(&cur);
        if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
        void *ptr = nullptr;
        if (e == hipSuccess) e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) {
            g_last_hip_error = (int)e;
            return DG_ERR_HIP;
        }
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return 0;
}

}  // namespace

extern "C" {

int dg_gemm(dg_op_t transA, dg_op_t transB, int64_t M, int64_t N, int64_t K, float alpha, const void *A,
            int64_t lda, const void *B, int64_t ldb, float beta, void *C, int64_t ldc, dg_dtype_t dtype,
            void *stream)
{
    return run(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, dtype, stream,
               DG_KERNEL_AUTO);
}

int dg_gemm_with_kernel(dg_op_t transA, dg_op_t transB, int64_t M, int64_t N, int64_t K, float alpha,
                        const void *A, int64_t lda, const void *B, int64_t ldb, float beta,
                        void *C, int64_t ldc, dg_dtype_t dtype, void *stream, int kernel)
{
    return run(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, dtype, stream,
               kernel);
}

int dg_gemm_ex(dg_op_t transA, dg_op_t transB, int64_t M, int64_t N, int64_t K, float alpha,
               const void *A, int64_t lda, int64_t strideA, const void *B, int64_t ldb,
               int64_t strideB, float beta, void *C, int64_t ldc, int64_t strideC,
               int64_t batch, const void *bias, dg_epilogue_t epilogue, dg_dtype_t dtype, void *stream)
{
    return dg_gemm_ex_with_kernel(transA, transB, M, N, K, alpha, A, lda, strideA, B, ldb,
                                  strideB, beta, C, ldc, strideC, batch, bias, epilogue, dtype,
                                  stream, DG_KERNEL_AUTO);
}

int dg_gemm_ex_with_kernel(dg_op_t transA, dg_op_t transB, int64_t M, int64_t N, int64_t K, float alpha,
                           const void *A, int64_t lda, int64_t strideA, const void *B,
                           int64_t ldb, int64_t strideB, float beta, void *C, int64_t ldc,
                           int64_t strideC, int64_t batch, const void *bias,
                           dg_epilogue_t epilogue, dg_dtype_t dtype, void *stream, int kernel)
{
    Ext x;
    x.sA = strideA;
    x.sB = strideB;
    x.sC = strideC;
    x.batch = batch;
    x.bias = bias;
    x.act = epilogue;
    int rc = validate(transA, transB, M, N, K, alpha, A, lda, B, ldb, C, ldc, dtype,
                      batch > 0);
    if (rc) return ex_position(rc);
    rc = validate_ext(M, N, ldc, x, dtype);
    if (rc) return rc;
    rc = run(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, dtype, stream, kernel,
             1, nullptr, 0, x);
    return rc < 0 && rc > -100 ? ex_position(rc) : rc;
}

int dg_gemm_splitk(dg_op_t transA, dg_op_t transB, int64_t M, int64_t N, int64_t K, float alpha,
                   const void *A, int64_t lda, const void *B, int64_t ldb, float beta, void *C,
                   int64_t ldc, dg_dtype_t dtype, void *stream, int splits, void *workspace,
                   size_t workspace_bytes)
{
    int rc = validate(transA, transB, M, N, K, alpha, A, lda, B, ldb, C, ldc, dtype);
    if (rc) return rc;
    if (splits < 0 || splits > 4096) return -16;
    if (splits != 1 && M > 0 && N > 0 && (workspace == nullptr || !aligned16(workspace))) return -17;
    return run(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, dtype, stream,
               DG_KERNEL_AUTO, splits, workspace, workspace_bytes);
}

int dg_gemm_splitk_noalloc(dg_op_t transA, dg_op_t transB, int64_t M, int64_t N, int64_t K,
                           float alpha, const void *A, int64_t lda, const void *B, int64_t ldb,
                           float beta, void *C, int64_t ldc, dg_dtype_t dtype, void *stream,
                           int splits)
{
    int rc = validate(transA, transB, M, N, K, alpha, A, lda, B, ldb, C, ldc, dtype);
    if (rc) return rc;
    if (splits < 0 || splits > 4096) return -16;
    if (M == 0 || N == 0) return DG_OK;
    // the ranges dg_gemm_splitk would use; more partials than the scratch
    // holds are refused before anything is enqueued
    int used = 1;
    if (K > 0 && alpha != 0.f) {
        const int k = choose(transA, transB, M, N, K, A, lda, B, ldb, dtype, Ext(),
                             c_rows_vec(C, ldc, dtype, Ext()));
        int32_t chunk;
        used = resolve_splits(kFamilies[k], M, N, K, splits, &chunk);
    }
    void *ws = nullptr;
    if (used > 1) {
        if ((size_t)used * (size_t)M * (size_t)N * 4 > (size_t)DG_SCRATCH_BYTES) return DG_ERR_SCRATCH;
        rc = scratch_for(stream, &ws);
        if (rc) return rc;
    }
    return run(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, dtype, stream,
               DG_KERNEL_AUTO, used > 1 ? splits : 1, ws, (size_t)DG_SCRATCH_BYTES);
}

int dg_gemm_splitk_choose(dg_op_t transA, dg_op_t transB, int64_t M, int64_t N, int64_t K,
                          dg_dtype_t dtype)
{
    int rc = validate(transA, transB, M, N, K, 1.f, nullptr, transA ? (M > 1 ? M : 1) : (K > 1 ? K : 1),
                      nullptr, transB ? (K > 1 ? K : 1) : (N > 1 ? N : 1), nullptr, N > 1 ? N : 1,
                      dtype, false);
    if (rc) return rc;
    if (M == 0 || N == 0 || K == 0) return 1;
    // the tile of the kernel dg_gemm would pick for aligned operands
    const int k = choose(transA, transB, M, N, K, (const void *)256, transA ? ((M + 7) / 8) * 8 : ((K + 7) / 8) * 8,
                         (const void *)256, transB ? ((K + 7) / 8) * 8 : ((N + 7) / 8) * 8, dtype, Ext());
    const Family &f = kFamilies[k];
    if (f.kind == SIMPLE) return 1;
    return splits_for(ceil_div(M, f.bm) * ceil_div(N, f.bn), K);
}

size_t dg_gemm_splitk_workspace_size(int64_t M, int64_t N, int splits)
{
    if (M <= 0 || N <= 0 || splits <= 1) return 0;
    return (size_t)splits * (size_t)M * (size_t)N * 4;
}

int dg_select_kernel(dg_op_t transA, dg_op_t transB, int64_t M, int64_t N, int64_t K, const void *A,
                     int64_t lda, const void *B, int64_t ldb, const void *C, int64_t ldc,
                     dg_dtype_t dtype)
{
    int rc = validate(transA, transB, M, N, K, 1.f, A, lda, B, ldb, C, ldc, dtype, false);
    if (rc) return rc;
    return choose(transA, transB, M, N, K, A, lda, B, ldb, dtype, Ext(), c_rows_vec(C, ldc, dtype, Ext()));
}

int dg_kernel_count(void) { return kNumKernels; }

const char *dg_kernel_name(int kernel)
{
    return (kernel >= 0 && kernel < kNumKernels) ? kFamilies[kernel].name : nullptr;
}

int dg_kernel_tile_m(int kernel)
{
    return (kernel >= 0 && kernel < kNumKernels) ? kFamilies[kernel].bm : -1;
}

int dg_kernel_tile_n(int kernel)
{
    return (kernel >= 0 && kernel < kNumKernels) ? kFamilies[kernel].bn : -1;
}

const char *dg_status_string(int status)
{
    switch (status) {
    case DG_OK: return "ok";
    case DG_ERR_UNSUPPORTED: return "kernel does not support this problem";
    case DG_ERR_SCRATCH: return "split-K partials larger than the library's scratch (DG_SCRATCH_BYTES)";
    case DG_ERR_HIP: return "HIP error (see dg_last_hip_error)";
    case -1: return "invalid argument 1 (transA)";
    case -2: return "invalid argument 2 (transB)";
    case -3: return "invalid argument 3 (M)";
    case -4: return "invalid argument 4 (N)";
    case -5: return "invalid argument 5 (K)";
    case -6: return "invalid argument 6 (alpha)";
    case -7: return "invalid argument 7 (A is NULL)";
    case -8: return "invalid argument 8 (lda)";
    case -9: return "invalid argument 9 (B is NULL; dg_gemm_ex: strideA)";
    case -10: return "invalid argument 10 (ldb; dg_gemm_ex: B is NULL)";
    case -11: return "invalid argument 11 (beta; dg_gemm_ex: ldb)";
    case -12: return "invalid argument 12 (C is NULL; dg_gemm_ex: strideB)";
    case -13: return "invalid argument 13 (ldc; dg_gemm_ex: beta)";
    case -14: return "invalid argument 14 (dtype; dg_gemm_ex: C is NULL)";
    case -15: return "invalid argument 15 (stream; dg_gemm_ex: ldc)";
    case -16: return "invalid argument 16 (dg_gemm_splitk: splits; dg_gemm_ex: strideC overlaps batches)";
    case -17: return "invalid argument 17 (dg_gemm_splitk: workspace NULL or not 16-byte aligned; "
                     "dg_gemm_ex: batch)";
    case -18: return "invalid argument 18 (dg_gemm_splitk: workspace too small; dg_gemm_ex: bias "
                     "not aligned to its element)";
    case -19: return "invalid argument 19 (dg_gemm_ex: epilogue)";
    case -20: return "invalid argument 20 (dg_gemm_ex: dtype)";
    default: return "unknown status";
    }
}

int dg_last_hip_error(void) { return g_last_hip_error; }

int dg_version(void) { return 400; }

}  // extern "C"
