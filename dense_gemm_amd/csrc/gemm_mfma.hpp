// Matrix-core GEMM kernel template for gfx950 (CDNA4), 64-lane waves.
//
//   C[BM x BN tile] = act(alpha * sum_k op(A)[tile rows, k] op(B)[k, tile cols]
//                         + beta * C + bias[cols]), batch blockIdx.y of a strided batch
//
// Hierarchy (the tiling of "Optimizing GEMM on Apple's M5 from scratch",
// Part 1 Kernels 2-4 and Part 2 Kernels 6-7, recast for CDNA4):
//   workgroup: 256 threads = 4 waves, owns a BM x BN tile of C, walks K in
//              slabs of BK;
//   wave:      owns a WM x WN sub-tile = (WM/32) x (WN/32) blocks of 32 x 32;
//   block:     one MFMA accumulator (16 fp32 per lane), updated by
//              v_mfma_f32_32x32x2_f32 (fp32) or v_mfma_f32_32x32x16_f16
//              (fp16 operands, fp32 accumulators -- the accumulator type that
//              keeps the fast path, "Metal GEMM Kernels for LoRA Training",
//              section 1).
//
// Data movement per K slab (double-buffered LDS, one barrier per slab, the
// prefetch of "From a C loop to a GPU kernel", double-buffering section):
//   1. issue 16-byte global loads of slab k+1 into registers (lanes run along
//      each stored matrix's contiguous dimension, so a wave reads whole
//      cache lines);
//   2. read slab k from LDS in the MFMA operand layout and run the MFMAs;
//   3. write the registers of slab k+1 to the other LDS buffer;
//   4. barrier.
//
// LDS layouts.  fp32: each operand keeps its stored orientation in LDS
// (rows padded by 16 bytes); a k-contiguous operand is read 4 k-values per
// ds_read_b128, an m/n-contiguous one one value per ds_read_b32 with the 32
// lanes of a half-wave on consecutive m (or n).  fp16: the MFMA wants 8
// consecutive k per lane, so both operands are kept k-contiguous in LDS; an
// m/n-contiguous operand is transposed in registers on its way into LDS (the
// write-side transpose of "Metal GEMM Kernels for LoRA Training", section 3),
// so the fragment reads stay linear.
//
// K order inside a slab: lane half h (lane / 32) of step s takes slab column
// h*BK/2 + s (fp32) or h*BK/2 + 8s .. +7 (fp16) for both operands, so each
// lane reads a contiguous run of its row.  Any fixed assignment is a valid
// summation order.
//
// Edges: rows, columns and k beyond the matrix are loaded as zeros, stores are
// guarded, so any M, N, K works.  VEC = false replaces each 16-byte load by
// element loads, for strides or pointers that are not 16-byte aligned.
#pragma once

#include "gemm_common.hpp"

namespace dg {

template <typename T> struct ElemTraits;
template <> struct ElemTraits<float> {
    static constexpr int V = 4;  // elements per 16-byte vector
    typedef f32x4 vec;
};
template <> struct ElemTraits<_Float16> {
    static constexpr int V = 8;
    typedef f16x8 vec;
};
template <> struct ElemTraits<__bf16> {
    static constexpr int V = 8;
    typedef bf16x8 vec;
};

// Load V consecutive elements p[0 .. V-1]; elements at or beyond `valid` are
// zero and are not read.
template <typename T, bool VEC>
__device__ __forceinline__ typename ElemTraits<T>::vec load_vec(const T *p, int valid)
{
    typedef typename ElemTraits<T>::vec vec;
    constexpr int V = ElemTraits<T>::V;
    vec v;
    if (VEC && valid >= V) {
        v = *(const vec *)p;
    } else {
#pragma unroll
        for (int e = 0; e < V; ++e) {
            T x = (T)0.f;
            if (e < valid) x = p[e];
            v[e] = x;
        }
    }
    return v;
}

// ---------------------------------------------------------------------------
// One operand's slab: BMN rows of op(A) (or columns of op(B)) by BK of k.
//   KCONT: the stored matrix has k contiguous (A not transposed, B transposed).
// ---------------------------------------------------------------------------
template <typename T, int BMN, int BK, bool KCONT, bool VEC>
struct Operand {
    static constexpr int V = ElemTraits<T>::V;
    typedef typename ElemTraits<T>::vec vec;
    static constexpr bool F16 = sizeof(T) == 2;
    // LDS layout
    static constexpr bool LDS_KMAJOR = KCONT || F16;  // rows = mn, k contiguous
    static constexpr int LD = LDS_KMAJOR ? (BK + V) : (BMN + V);
    static constexpr int ELEMS = LDS_KMAJOR ? BMN * LD : BK * LD;
    // global -> register mapping
    static constexpr int PER_THREAD = BMN * BK / 256;  // elements
    static constexpr int NV = PER_THREAD / V;           // 16-byte vectors per thread
    static_assert(NV * V * 256 == BMN * BK, "tile must split into 16-byte vectors");
    // KCONT: lanes along k
    static constexpr int LPR = BK / V;          // lanes per row
    static constexpr int RPP = 256 / LPR;       // rows per pass
    // !KCONT: lanes along mn
    static constexpr int LPK = BMN / V;         // lanes per k row
    static constexpr int KG = 256 / LPK;        // k groups
    static constexpr int KV = BK / KG;          // consecutive k rows per thread (fp16 transpose)

    vec r[NV];

    // Global loads of the slab starting at (mn0, k0).  ext = rows of op(A) (M)
    // or columns of op(B) (N).
    __device__ __forceinline__ void load(const T *g, int64_t ld, int mn0, int k0, int ext, int K,
                                         int tid)
    {
        if constexpr (KCONT) {
            const int rr = tid / LPR, c = (tid % LPR) * V;
#pragma unroll
            for (int q = 0; q < NV; ++q) {
                const int mn = mn0 + q * RPP + rr, k = k0 + c;
                const int valid = (mn < ext) ? (K - k) : 0;
                r[q] = load_vec<T, VEC>(g + (int64_t)mn * ld + k, valid);
            }
        } else if constexpr (!F16) {
            // fp32, stored k x mn: passes over k rows, lanes along mn
            const int kr = tid / LPK, c = (tid % LPK) * V;
#pragma unroll
            for (int q = 0; q < NV; ++q) {
                const int k = k0 + q * KG + kr, mn = mn0 + c;
                const int valid = (k < K) ? (ext - mn) : 0;
                r[q] = load_vec<T, VEC>(g + (int64_t)k * ld + mn, valid);
            }
        } else {
            // fp16, stored k x mn: KV consecutive k rows per thread, to be
            // transposed into k-contiguous runs
            static_assert(KV * KG == BK && NV == KV, "fp16 transpose mapping");
            const int kg = tid / LPK, c = (tid % LPK) * V;
#pragma unroll
            for (int q = 0; q < NV; ++q) {
                const int k = k0 + kg * KV + q, mn = mn0 + c;
                const int valid = (k < K) ? (ext - mn) : 0;
                r[q] = load_vec<T, VEC>(g + (int64_t)k * ld + mn, valid);
            }
        }
    }

    __device__ __forceinline__ void store(T *s, int tid) const
    {
        if constexpr (KCONT) {
            const int rr = tid / LPR, c = (tid % LPR) * V;
#pragma unroll
            for (int q = 0; q < NV; ++q)
                *(vec *)(s + (q * RPP + rr) * LD + c) = r[q];
        } else if constexpr (!F16) {
            const int kr = tid / LPK, c = (tid % LPK) * V;
#pragma unroll
            for (int q = 0; q < NV; ++q)
                *(vec *)(s + (q * KG + kr) * LD + c) = r[q];
        } else {
            // register transpose: column j of the KV x V block becomes a run
            // of KV k-values in LDS row (c + j)
            const int kg = tid / LPK, c = (tid % LPK) * V;
            typedef T run_t __attribute__((ext_vector_type(KV)));
#pragma unroll
            for (int j = 0; j < V; ++j) {
                run_t t;
#pragma unroll
                for (int q = 0; q < KV; ++q)
                    t[q] = r[q][j];
                *(run_t *)(s + (c + j) * LD + kg * KV) = t;
            }
        }
    }
};

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------
template <typename T, int BM, int BN, int BK, int WM, int WN, bool TA, bool TB, bool VEC, int MINW,
          typename TC = T>
__global__ __launch_bounds__(256, MINW) void gemm_mfma_kernel(GemmParams p)
{
    constexpr bool F16 = sizeof(T) == 2;
    constexpr int WAVES_N = BN / WN;
    static_assert((BM / WM) * WAVES_N == 4, "4 waves per workgroup");
    constexpr int TM = WM / 32, TN = WN / 32;
    typedef Operand<T, BM, BK, !TA, VEC> OpA;  // A k-contiguous unless transposed
    typedef Operand<T, BN, BK, TB, VEC> OpB;   // B k-contiguous only when transposed
    constexpr int STAGE = OpA::ELEMS + OpB::ELEMS;
    __shared__ __attribute__((aligned(16))) T smem[2 * STAGE];

    select_batch<T, TC>(p, blockIdx.y);
    int bid, split, k_begin, Kl;
    split_of(p, bid, split, k_begin, Kl);
    // this split's k range starts at k_begin: offset the operands to it
    const T *A = (const T *)p.A + (TA ? (int64_t)k_begin * p.lda : (int64_t)k_begin);
    const T *B = (const T *)p.B + (TB ? (int64_t)k_begin : (int64_t)k_begin * p.ldb);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm0 = (wave / WAVES_N) * WM;
    const int wn0 = (wave % WAVES_N) * WN;
    int tm, tn;
    tile_coords(bid, p, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int nk = (Kl + BK - 1) / BK;

    OpA ga;
    OpB gb;
    ga.load(A, p.lda, m0, 0, p.M, Kl, tid);
    gb.load(B, p.ldb, n0, 0, p.N, Kl, tid);
    ga.store(smem, tid);
    gb.store(smem + OpA::ELEMS, tid);
    __syncthreads();

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.f;

    const int lrow = lane & 31;          // row (m or n) inside a 32-block
    const int khalf = (lane >> 5) * (BK / 2);  // this lane half's k range in the slab

    for (int kt = 0; kt < nk; ++kt) {
        const T *sA = smem + (kt & 1) * STAGE;
        const T *sB = sA + OpA::ELEMS;
        const bool more = kt + 1 < nk;
        if (more) {
            ga.load(A, p.lda, m0, (kt + 1) * BK, p.M, Kl, tid);
            gb.load(B, p.ldb, n0, (kt + 1) * BK, p.N, Kl, tid);
        }
        if constexpr (!F16) {
            // fp32: 32x32x2 MFMA, BK/2 steps; 4 steps per chunk
#pragma unroll
            for (int c = 0; c < BK / 8; ++c) {
                float a[TM][4], b[TN][4];
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    if constexpr (OpA::LDS_KMAJOR) {
                        const f32x4 v = *(const f32x4 *)(sA + (wm0 + 32 * i + lrow) * OpA::LD + khalf + 4 * c);
#pragma unroll
                        for (int e = 0; e < 4; ++e) a[i][e] = v[e];
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            a[i][e] = sA[(khalf + 4 * c + e) * OpA::LD + wm0 + 32 * i + lrow];
                    }
                }
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    if constexpr (OpB::LDS_KMAJOR) {
                        const f32x4 v = *(const f32x4 *)(sB + (wn0 + 32 * j + lrow) * OpB::LD + khalf + 4 * c);
#pragma unroll
                        for (int e = 0; e < 4; ++e) b[j][e] = v[e];
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            b[j][e] = sB[(khalf + 4 * c + e) * OpB::LD + wn0 + 32 * j + lrow];
                    }
                }
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int j = 0; j < TN; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][e], b[j][e], acc[i][j], 0, 0, 0);
            }
        } else {
            // fp16: 32x32x16 MFMA, BK/16 steps, 8 k per lane per step
#pragma unroll
            for (int c = 0; c < BK / 16; ++c) {
                typedef typename ElemTraits<T>::vec v8;
                v8 a[TM], b[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    a[i] = *(const v8 *)(sA + (wm0 + 32 * i + lrow) * OpA::LD + khalf + 8 * c);
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    b[j] = *(const v8 *)(sB + (wn0 + 32 * j + lrow) * OpB::LD + khalf + 8 * c);
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = mfma_32x32x16(a[i], b[j], acc[i][j]);
            }
        }
        if (more) {
            T *s = smem + ((kt + 1) & 1) * STAGE;
            ga.store(s, tid);
            gb.store(s + OpA::ELEMS, tid);
        }
        __syncthreads();
    }

    // Epilogue.  Accumulator register r of lane l in a 32x32 block holds
    // row 8*(r/4) + 4*(l/32) + r%4, column l%32: for a fixed r the 32 lanes
    // of a half-wave hold 32 consecutive columns of one row.
    TC *C = (TC *)p.C;
    const int lcol = lane & 31;
    const int lrow4 = (lane >> 5) * 4;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int col = n0 + wn0 + 32 * j + lcol;
            if (col >= p.N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm0 + 32 * i + 8 * (r >> 2) + lrow4 + (r & 3);
                if (row < p.M && p.splits > 1) {
                    p.ws[((int64_t)split * p.M + row) * p.N + col] = acc[i][j][r];
                } else if (row < p.M) {
                    TC *c = C + (int64_t)row * p.ldc + col;
                    const float cin = p.beta != 0.f ? (float)*c : 0.f;
                    *c = (TC)epilogue_value<TC>(p, acc[i][j][r], cin, col);
                }
            }
        }
    }
}

template <typename T, int BM, int BN, int BK, int WM, int WN, bool TA, bool TB, bool VEC, int MINW,
          typename TC = T>
hipError_t launch_mfma(const GemmParams &p, hipStream_t s)
{
    const unsigned nwg = (unsigned)p.tiles_m * (unsigned)p.tiles_n * (unsigned)(p.splits > 1 ? p.splits : 1);
    GemmParams arg = p;
    void *args[] = {&arg};
    return hipLaunchKernel((const void *)&gemm_mfma_kernel<T, BM, BN, BK, WM, WN, TA, TB, VEC, MINW, TC>,
                           dim3(nwg, p.batch), dim3(256), args, 0, s);
}

}  // namespace dg
