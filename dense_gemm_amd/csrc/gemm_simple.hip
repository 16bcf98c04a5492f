// Generic GEMM kernel: any shape, any leading dimension, any alignment, all
// four transpose pairs, fp32, fp16 or bf16 operands, fp32 accumulation, an
// output of the operand type or fp32, the bias + activation epilogue and
// strided batches (grid z).
//
// Structure: the shared-memory tiling of "Optimizing GEMM on Apple's M5 from
// scratch, Part 1" (Kernels 2 and 3: stage a tile of each operand on chip,
// one barrier after the stores and one before they are overwritten) with the
// 2x2-per-thread register blocking idea of "From a C loop to a GPU kernel"
// (GPU tiling section) widened to 4x4, and the zero-filled masked edge loads
// and guarded stores of that page's tiled kernel.  Each element is loaded on
// its own, so no alignment is assumed; lanes run along whichever dimension
// the stored matrix has contiguous.
//
// This is the fallback for problems the matrix-core kernels do not take; the
// other kernels here serve the case without a product (alpha == 0 or K == 0)
// and the split-K reduction.
#include "gemm_common.hpp"

namespace dg {

namespace {

constexpr int ST = 64;   // output tile (ST x ST)
constexpr int SK = 16;   // K slab
constexpr int SPAD = 4;

template <typename T>
__device__ __forceinline__ float to_f32(T v) { return (float)v; }

template <typename T, bool TA, bool TB, typename TC>
__global__ __launch_bounds__(256) void gemm_simple_kernel(GemmParams p)
{
    __shared__ float As[SK][ST + SPAD];
    __shared__ float Bs[SK][ST + SPAD];
    select_batch<T, TC>(p, blockIdx.z);
    const T *A = (const T *)p.A;
    const T *B = (const T *)p.B;
    TC *C = (TC *)p.C;
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    const int m0 = blockIdx.y * ST, n0 = blockIdx.x * ST;
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = 0.f;

    for (int k0 = 0; k0 < p.K; k0 += SK) {
#pragma unroll
        for (int q = 0; q < (ST * SK) / 256; ++q) {
            const int e = tid + q * 256;
            int mm, kk;
            if (TA) { kk = e / ST; mm = e % ST; }   // stored K x M: lanes along m
            else    { mm = e / SK; kk = e % SK; }   // stored M x K: lanes along k
            const int gm = m0 + mm, gk = k0 + kk;
            float v = 0.f;
            if (gm < p.M && gk < p.K)
                v = to_f32(TA ? A[(int64_t)gk * p.lda + gm] : A[(int64_t)gm * p.lda + gk]);
            As[kk][mm] = v;
        }
#pragma unroll
        for (int q = 0; q < (ST * SK) / 256; ++q) {
            const int e = tid + q * 256;
            int nn, kk;
            if (TB) { nn = e / SK; kk = e % SK; }   // stored N x K: lanes along k
            else    { kk = e / ST; nn = e % ST; }   // stored K x N: lanes along n
            const int gn = n0 + nn, gk = k0 + kk;
            float v = 0.f;
            if (gn < p.N && gk < p.K)
                v = to_f32(TB ? B[(int64_t)gn * p.ldb + gk] : B[(int64_t)gk * p.ldb + gn]);
            Bs[kk][nn] = v;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < SK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int gm = m0 + ty * 4 + i;
        if (gm >= p.M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int gn = n0 + tx * 4 + j;
            if (gn >= p.N) continue;
            TC *c = C + (int64_t)gm * p.ldc + gn;
            const float cin = p.beta != 0.f ? to_f32(*c) : 0.f;
            *c = (TC)epilogue_value<TC>(p, acc[i][j], cin, gn);
        }
    }
}

// No product term (alpha == 0 or K == 0): C = act(beta * C + bias) over the
// M x N view of batch blockIdx.y; beta == 0 does not read C.
template <typename T>
__global__ __launch_bounds__(256) void scale_c_kernel(GemmParams p)
{
    select_batch<T>(p, blockIdx.y);
    T *C = (T *)p.C;
    const int64_t total = (int64_t)p.M * p.N;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * 256) {
        const int64_t i = e / p.N, j = e - i * p.N;
        T *c = C + i * p.ldc + j;
        float v = p.beta != 0.f ? p.beta * to_f32(*c) : 0.f;
        if (p.bias) v += to_f32(((const T *)p.bias)[j]);
        *c = (T)activate(p.act, v);
    }
}

// Split-K reduction (the second kernel of dg_gemm_splitk): C =
// act(alpha * sum_s ws[s] + beta * C + bias), the splits summed in increasing
// s (reduce_group4).  A thread takes 4 consecutive columns of one row; a row
// has 2^tpr_log2 threads (enough to cover N / 4 groups, at most 256), a
// workgroup 256 >> tpr_log2 rows, so the row and column come from shifts.
template <typename T>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmParams p, int tpr_log2)
{
    const int tpr = 1 << tpr_log2;
    const int64_t row = (int64_t)blockIdx.x * (256 >> tpr_log2) + (threadIdx.x >> tpr_log2);
    if (row >= p.M) return;
    for (int c0 = (threadIdx.x & (tpr - 1)) * 4; c0 < p.N; c0 += tpr * 4) reduce_group4<T>(p, row, c0);
}

template <typename T>
hipError_t launch_splitk_reduce(const GemmParams &p, hipStream_t s)
{
    const int64_t groups = ((int64_t)p.N + 3) / 4;            // 4-column groups per row
    int tpr_log2 = 0;
    while (tpr_log2 < 8 && ((int64_t)1 << tpr_log2) < groups) ++tpr_log2;
    const int64_t rows_per_block = 256 >> tpr_log2;
    const int64_t blocks = ((int64_t)p.M + rows_per_block - 1) / rows_per_block;
    GemmParams arg = p;
    int tl = tpr_log2;
    void *args[] = {&arg, &tl};
    return hipLaunchKernel((const void *)&splitk_reduce_kernel<T>, dim3((unsigned)blocks), dim3(256),
                           args, 0, s);
}

template <typename T, bool TA, bool TB, typename TC = T>
hipError_t launch_simple(const GemmParams &p, hipStream_t s)
{
    dim3 grid((p.N + ST - 1) / ST, (p.M + ST - 1) / ST, p.batch);
    GemmParams arg = p;
    void *args[] = {&arg};
    return hipLaunchKernel((const void *)&gemm_simple_kernel<T, TA, TB, TC>, grid, dim3(256), args, 0, s);
}

template <typename T>
hipError_t launch_scale(const GemmParams &p, hipStream_t s)
{
    const int64_t total = (int64_t)p.M * p.N;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    GemmParams arg = p;
    void *args[] = {&arg};
    return hipLaunchKernel((const void *)&scale_c_kernel<T>, dim3((unsigned)blocks, p.batch), dim3(256),
                           args, 0, s);
}

}  // namespace

// launchers exported to the dispatcher, indexed by the dtype of the C ABI:
// 0 fp32; 1 fp16 -> fp16; 2 bf16 -> bf16; 3 fp16 -> fp32; 4 bf16 -> fp32.
// [dtype][transA][transB]
launch_fn simple_launcher(int dtype, int ta, int tb)
{
#define DG_SIMPLE4(T, TC)                                                                          \
    {{launch_simple<T, false, false, TC>, launch_simple<T, false, true, TC>},                      \
     {launch_simple<T, true, false, TC>, launch_simple<T, true, true, TC>}}
    static const launch_fn table[5][2][2] = {
        DG_SIMPLE4(float, float), DG_SIMPLE4(_Float16, _Float16), DG_SIMPLE4(__bf16, __bf16),
        DG_SIMPLE4(_Float16, float), DG_SIMPLE4(__bf16, float),
    };
#undef DG_SIMPLE4
    return table[dtype][ta][tb];
}

// The reduction and the scale kernel touch only C (and the bias): they go by
// the output type.
launch_fn splitk_reduce_launcher(int dtype)
{
    static const launch_fn table[5] = {launch_splitk_reduce<float>, launch_splitk_reduce<_Float16>,
                                       launch_splitk_reduce<__bf16>, launch_splitk_reduce<float>,
                                       launch_splitk_reduce<float>};
    return table[dtype];
}

launch_fn scale_launcher(int dtype)
{
    static const launch_fn table[5] = {launch_scale<float>, launch_scale<_Float16>, launch_scale<__bf16>,
                                       launch_scale<float>, launch_scale<float>};
    return table[dtype];
}

}  // namespace dg
