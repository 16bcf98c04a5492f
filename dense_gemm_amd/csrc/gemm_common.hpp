// Internal declarations shared by the GEMM kernels and the host dispatcher of
// libdense_gemm_amd.so (gfx950).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Everything a kernel needs for one C = alpha*op(A)*op(B) + beta*C.
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
};

// A host-side launcher: enqueues one kernel on `stream`, returns a hipError_t.
typedef hipError_t (*launch_fn)(const GemmParams &p, hipStream_t stream);

#ifdef __HIPCC__
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
