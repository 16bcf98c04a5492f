// Internal declarations shared by the GEMM kernels and the host dispatcher of
// libdense_gemm_amd.so (gfx950).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// The 32x32x16 matrix-core step for either 16-bit operand type (fp32 accumulators).
__device__ __forceinline__ f32x16 mfma_32x32x16(f16x8 a, f16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Epilogue activations (the values of dg_gemm_ex's `epilogue`).
enum { ACT_NONE = 0, ACT_RELU = 1, ACT_GELU = 2 };

// Everything a kernel needs for one act(alpha*op(A)*op(B) + beta*C + bias),
// or a strided batch of them.  A and B hold the operand type; C and the bias
// hold the output type (the operand type, or fp32 for 16-bit operands with
// an fp32 output).
struct GemmParams {
    const void *A;
    const void *B;
    void *C;
    int64_t lda, ldb, ldc;  // row strides of the stored matrices (elements)
    int32_t M, N, K;        // op(A) is M x K, op(B) is K x N
    float alpha, beta;
    int32_t tiles_m, tiles_n;  // output tiles of the launch
    int32_t group_m;           // tile rows walked together (cache locality)
    int32_t c_vec;             // C rows start on 4-byte boundaries (16-byte accesses allowed)
    // split-K: with splits > 1 the grid is tiles x splits; workgroup (tile, s)
    // covers k in [s*k_chunk, min(K, (s+1)*k_chunk)) and writes its raw fp32
    // sums to ws[s][M][N] (row stride N) instead of C.
    int32_t splits;
    int32_t k_chunk;           // a multiple of every kernel's K slab
    float *ws;
    // epilogue: bias[col] (N elements of C's type, NULL for none) is added
    // after alpha and beta, then the activation `act` is applied
    const void *bias;
    int32_t act;
    // strided batch: batch b (a grid dimension) uses A + b*strideA,
    // B + b*strideB, C + b*strideC (elements); batch >= 1
    int64_t strideA, strideB, strideC;
    int32_t batch;
};

// A host-side launcher: enqueues one kernel on `stream`, returns a hipError_t.
typedef hipError_t (*launch_fn)(const GemmParams &p, hipStream_t stream);

#ifdef __HIPCC__
// Point A, B (elements of type T) and C (elements of type TC) at batch b.
template <typename T, typename TC = T>
__device__ __forceinline__ void select_batch(GemmParams &p, int b)
{
    p.A = (const T *)p.A + (int64_t)b * p.strideA;
    p.B = (const T *)p.B + (int64_t)b * p.strideB;
    p.C = (TC *)p.C + (int64_t)b * p.strideC;
}

// gelu(x) = x * Phi(x), Phi(x) = (1 + erf(x / sqrt 2)) / 2, in fp32.  erf by
// the rational approximation of Abramowitz & Stegun, Handbook of
// Mathematical Functions, eq. 7.1.26 (after Hastings): for z >= 0,
//   erfc(z) = (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-z^2),
//   t = 1 / (1 + p z), |error| <= 1.5e-7.
// With q = erfc(|x| / sqrt 2): gelu = x (1 - q/2) for x >= 0 and x q / 2 for
// x < 0, so the negative side never forms 1 - erf and keeps its relative
// accuracy.  About a dozen instructions against a general erff's several
// dozen, which matters because the epilogue runs once per output after the
// K loop, with nothing to overlap it.
__device__ __forceinline__ float gelu(float x)
{
    const float z = __builtin_fabsf(x) * 0.70710678118654752f;
    const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.3275911f, z, 1.f));
    float poly = __builtin_fmaf(t, 1.061405429f, -1.453152027f);
    poly = __builtin_fmaf(t, poly, 1.421413741f);
    poly = __builtin_fmaf(t, poly, -0.284496736f);
    poly = __builtin_fmaf(t, poly, 0.254829592f);
    const float q = poly * t * __expf(-z * z);
    return x >= 0.f ? x * __builtin_fmaf(-0.5f, q, 1.f) : 0.5f * x * q;
}

// The activation of the epilogue, in fp32.  relu keeps NaN (the comparison
// is false for it); gelu as above (NaN stays NaN).
__device__ __forceinline__ float activate(int act, float x)
{
    if (act == ACT_RELU) return x < 0.f ? 0.f : x;
    if (act == ACT_GELU) return gelu(x);
    return x;
}

// Everything after the accumulation for one output element: v = alpha*acc
// (+ beta*c_in when beta != 0) + bias[col], then the activation, in fp32.
template <typename T>
__device__ __forceinline__ float epilogue_value(const GemmParams &p, float acc, float c_in, int col)
{
    float v = p.alpha * acc;
    if (p.beta != 0.f) v = __builtin_fmaf(p.beta, c_in, v);
    if (p.bias) v += (float)((const T *)p.bias)[col];
    return activate(p.act, v);
}

// The same for W consecutive columns col .. col+W-1 (all < N): the bias is
// read with vector loads (16 bytes, or the W elements when they are fewer)
// when its address allows.
template <typename T, int W>
__device__ __forceinline__ void epilogue_row(const GemmParams &p, float (&v)[W], const float (&cin)[W], int col)
{
    constexpr int PER = (int)(16 / sizeof(T)) < W ? (int)(16 / sizeof(T)) : W;  // elements per bias load
    float b[W];
#pragma unroll
    for (int e = 0; e < W; ++e) b[e] = 0.f;
    if (p.bias) {
        const T *bp = (const T *)p.bias + col;
        if (((uintptr_t)bp & (PER * sizeof(T) - 1)) == 0) {
            typedef T VT __attribute__((ext_vector_type(PER)));
#pragma unroll
            for (int c = 0; c < W / PER; ++c) {
                const VT x = *(const VT *)(bp + c * PER);
#pragma unroll
                for (int e = 0; e < PER; ++e) b[c * PER + e] = (float)x[e];
            }
        } else {
#pragma unroll
            for (int e = 0; e < W; ++e) b[e] = (float)bp[e];
        }
    }
#pragma unroll
    for (int e = 0; e < W; ++e) {
        float x = p.alpha * v[e];
        if (p.beta != 0.f) x = __builtin_fmaf(p.beta, cin[e], x);
        v[e] = activate(p.act, x + b[e]);
    }
}

template <typename T>
__device__ __forceinline__ void epilogue_row16(const GemmParams &p, float (&v)[16], const float (&cin)[16],
                                               int col)
{
    epilogue_row<T, 16>(p, v, cin, col);
}

// Split-K reduction of 4 consecutive columns c0 .. c0+3 of row `row` (only
// those below N): the splits' fp32 partials (ws[s] is M x N, row stride N)
// summed in increasing s starting from zero, then alpha, beta, bias and the
// activation in fp32 and one rounding to T.  beta == 0 does not read C.
// Partials are read with 16-byte loads when N is a multiple of 4 (the
// workspace is 16-byte aligned), eight splits' loads in flight at once; C is
// written with one vector store when its rows allow.
template <typename T>
__device__ __forceinline__ void reduce_group4(const GemmParams &p, int64_t row, int c0)
{
    typedef T V4 __attribute__((ext_vector_type(4)));
    const int64_t mn = (int64_t)p.M * p.N;
    const float *wcol = p.ws + row * p.N + c0;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    const bool full = c0 + 4 <= p.N;
    if (full && (p.N & 3) == 0) {
        for (int sp = 0; sp < p.splits; sp += 8) {
            // up to eight loads issued before the in-order sums
            f32x4 x[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (sp + u < p.splits) x[u] = *(const f32x4 *)(wcol + (sp + u) * mn);
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (sp + u < p.splits)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[e] += x[u][e];
        }
    } else {
        for (int sp = 0; sp < p.splits; ++sp)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (c0 + e < p.N) acc[e] += wcol[sp * mn + e];
    }
    T *c = (T *)p.C + row * p.ldc + c0;
    if (full && p.c_vec) {
        // rows start on 16-byte boundaries and c0 is a multiple of 4
        float cin[4] = {0.f, 0.f, 0.f, 0.f};
        if (p.beta != 0.f) {
            const V4 ci = *(const V4 *)c;
#pragma unroll
            for (int e = 0; e < 4; ++e) cin[e] = (float)ci[e];
        }
        epilogue_row<T, 4>(p, acc, cin, c0);
        V4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (T)acc[e];
        *(V4 *)c = o;
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (c0 + e < p.N) {
                const float cin = p.beta != 0.f ? (float)c[e] : 0.f;
                c[e] = (T)epilogue_value<T>(p, acc[e], cin, c0 + e);
            }
        }
    }
}

// Workgroup id -> (split, id of the tile within the split) and the split's
// k range [k_begin, k_begin + k_len).
__device__ __forceinline__ void split_of(const GemmParams &p, int &bid, int &split, int &k_begin,
                                         int &k_len)
{
    bid = blockIdx.x;
    split = 0;
    k_begin = 0;
    k_len = p.K;
    if (p.splits > 1) {
        const int ntiles = p.tiles_m * p.tiles_n;
        split = bid / ntiles;
        bid -= split * ntiles;
        k_begin = split * p.k_chunk;
        k_len = p.K - k_begin < p.k_chunk ? p.K - k_begin : p.k_chunk;
    }
}

// Workgroup id -> output tile (tm, tn).
//
// The hardware hands consecutive workgroup ids to the 8 XCDs in turn
// (id % 8), and each XCD has its own L2.  First undo that round-robin so
// that a contiguous range of "logical" ids runs on one XCD, then walk the
// logical ids group_m tile rows at a time (column-major inside the group), so
// that the tiles resident on one XCD share rows of op(A) and columns of op(B).
__device__ __forceinline__ void tile_coords(int bid, const GemmParams &p, int &tm, int &tn)
{
    const int nwg = p.tiles_m * p.tiles_n;
    const int xcd = bid & 7;
    const int local = bid >> 3;
    const int per = nwg >> 3;
    const int rem = nwg & 7;
    const int logical = xcd * per + (xcd < rem ? xcd : rem) + local;
    const int gsz = p.group_m * p.tiles_n;
    const int g = logical / gsz;
    const int first_m = g * p.group_m;
    const int rows = (p.tiles_m - first_m) < p.group_m ? (p.tiles_m - first_m) : p.group_m;
    const int in_g = logical - g * gsz;
    tm = first_m + in_g % rows;
    tn = in_g / rows;
}
#endif

}  // namespace dg
