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

// Epilogue activations (the values of dg_gemm_ex's `epilogue`).
enum { ACT_NONE = 0, ACT_RELU = 1, ACT_GELU = 2 };

// Everything a kernel needs for one act(alpha*op(A)*op(B) + beta*C + bias),
// or a strided batch of them.
struct GemmParams {
    const void *A;
    const void *B;
    void *C;
    int64_t lda, ldb, ldc;  // row strides of the stored matrices (elements)
    int32_t M, N, K;        // op(A) is M x K, op(B) is K x N
    float alpha, beta;
    int32_t tiles_m, tiles_n;  // output tiles of the launch
    int32_t group_m;           // tile rows walked together (cache locality)
    int32_t c_vec;             // C rows start on 16-byte boundaries (16-byte stores allowed)
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
// Point A, B and C at batch b.
template <typename T>
__device__ __forceinline__ void select_batch(GemmParams &p, int b)
{
    p.A = (const T *)p.A + (int64_t)b * p.strideA;
    p.B = (const T *)p.B + (int64_t)b * p.strideB;
    p.C = (T *)p.C + (int64_t)b * p.strideC;
}

// The activation of the epilogue, in fp32.  relu keeps NaN (the comparison
// is false for it); gelu is x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)) with the
// device erff.
__device__ __forceinline__ float activate(int act, float x)
{
    if (act == ACT_RELU) return x < 0.f ? 0.f : x;
    if (act == ACT_GELU) return 0.5f * x * (1.f + erff(x * 0.7071067811865476f));
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
