// Control probes of the GEMM measurements (libdense_gemm_probe.so): the
// matrix-core peak with the shader clock under load, a plain device copy, and
// the per-slab work of the fp16 GEMM tile without the GEMM (direct loads and
// MFMAs apart and together).
// "Metal GEMM Kernels for LoRA Training on Apple Silicon", section 9: figures
// are trusted only while a control benchmark stays within 10% of its
// reference.  These kernels have exactly known costs, so they serve as that
// control beside the GEMM figures.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "../../include/dense_gemm_probe.h"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char_t;

thread_local int g_last_hip_error = 0;

constexpr int kThreads = 256;

// Each wave: `iters` rounds of 8 independent MFMAs (two waves per SIMD when
// two workgroups share a CU keep the matrix core busy).  The first wave of
// each workgroup stamps the loop with the shader clock (s_memtime) and the
// constant wall clock (s_memrealtime).  DGP_MFMA_F16_RANDOM takes its
// operands from four sets of pseudo-random fp16 values in [-1, 1) (a
// per-lane hash), a different pair of sets for each MFMA of a round, so the
// matrix core's inputs change every instruction as they do on real data.
template <int KIND>
__global__ __launch_bounds__(kThreads) void mfma_peak_kernel(int iters, float *sink, uint64_t *clocks)
{
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    f32x16 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t w0 = __builtin_amdgcn_s_memrealtime();
    if constexpr (KIND == DGP_MFMA_F16_RANDOM) {
        f16x8 a[4], b[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // a 32-bit integer hash (multiply-xorshift) of lane, set and element
                uint32_t h = (uint32_t)(((blockIdx.x * kThreads + tid) * 4 + q) * 16 + e) * 0x9E3779B1u;
                h ^= h >> 15;
                h *= 0x85EBCA77u;
                h ^= h >> 13;
                a[q][e] = (_Float16)((float)(h & 0xffff) * (1.0f / 32768.0f) - 1.0f);
                b[q][e] = (_Float16)((float)(h >> 16) * (1.0f / 32768.0f) - 1.0f);
            }
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i & 3], b[(i + (i >> 2)) & 3], acc[i], 0, 0, 0);
        }
    } else if constexpr (KIND == DGP_MFMA_F16) {
        f16x8 a, b;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            a[e] = (_Float16)(lane * 0.001f + e * 0.01f);
            b[e] = (_Float16)(e * 0.5f - 1.f);
        }
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[i], 0, 0, 0);
        }
    } else {
        const float a = lane * 0.001f, b = 0.5f;
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[i], 0, 0, 0);
        }
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t w1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[i][r];
    sink[(int64_t)blockIdx.x * kThreads + tid] = s;
    if (tid == 0) {
        clocks[2 * (int64_t)blockIdx.x] = t1 - t0;
        clocks[2 * (int64_t)blockIdx.x + 1] = w1 - w0;
    }
}

__global__ __launch_bounds__(kThreads) void copy_kernel(const i32x4 *src, i32x4 *dst, int64_t n16)
{
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

// The per-slab work of the 128x128 fp16 GEMM tile (two K groups of four
// waves, four 32 KB LDS stages, one workgroup per CU), without its data
// flow: each iteration is one slab.  It starts as a GEMM slab does (wait
// until this wave has at most two slabs' loads in flight, one with
// DGP_SLAB_DEPTH1, then a barrier); then each wave does the parts MODE names
// (DGP_SLAB_* bits):
//   LOADS  4 direct loads of 1 KB (buffer_load_dwordx4 ... lds, 16 bytes per
//          lane), 32 KB per workgroup: a window of 256 rows x 128 bytes of
//          `src`, seen as rows of `pitch` bytes (pitch 128: contiguous).
//          Workgroup ids are dealt to the 8 XCDs in turn; the workgroups of
//          one XCD share `windows` groups of 256 rows, the XCDs take
//          different groups, and slab i reads column i % (pitch / 128) of
//          its group, moving on to the next groups when the columns wrap,
//          as a GEMM tile walks K along its A and B panels.  With PANELS the
//          loads are exactly a GEMM tile's instead: workgroup w is tile
//          (tm, tn) of a T x T grid (T * T workgroups) in the library's
//          XCD-aware order with `windows` tile rows per group; its first 16
//          KB are rows tm*128 .. +128 of A (the first half of src), the
//          other 16 KB rows tn*128 .. +128 of B (the second half), one
//          128-byte column per slab, the columns wrapping.  With SWIZZLE
//          the 8 lanes of a row fetch its 16-byte chunks in the order the
//          fp16 GEMM's k-contiguous operand does (lane l: chunk
//          (l % 8) ^ ((row / 2) % 8)), not in address order;
//   MFMA   8 v_mfma_f32_32x32x16_f16 (16 per SIMD: the slab's matrix-core
//          work), on 2 x 2 blocks of two 16-deep k steps;
//   READS  8 fragment reads of 1 KB (ds_read_b128, 16 bytes per lane,
//          conflict-free), 64 KB per workgroup, from the stage loaded two
//          slabs earlier; with MFMA they are the next slab's operands, read
//          while this slab's MFMAs run, as the GEMM reads them.
// A load goes before every second MFMA step and a read before every one, in
// that order (pinned with sched_barrier).  Without READS the MFMAs take
// register operands; without MFMA the reads feed a sum.  The first wave
// stamps the loop with the shader clock (s_memtime) and the constant wall
// clock (s_memrealtime).
template <int MODE>
__global__ __launch_bounds__(512) void slab_probe_kernel(const char *src, uint32_t src_bytes, int iters,
                                                        int windows, uint32_t pitch, float *sink,
                                                        uint64_t *clocks)
{
    constexpr bool LOADS = (MODE & DGP_SLAB_LOADS) != 0;
    constexpr bool MFMA = (MODE & DGP_SLAB_MFMA) != 0;
    constexpr bool READS = (MODE & DGP_SLAB_READS) != 0;
    constexpr bool DEPTH1 = (MODE & DGP_SLAB_DEPTH1) != 0;
    constexpr bool PANELS = (MODE & DGP_SLAB_PANELS) != 0;
    constexpr bool SWIZZLE = (MODE & DGP_SLAB_SWIZZLE) != 0;
    typedef __attribute__((address_space(3))) f16x8 lds_f16x8_t;
    __shared__ __attribute__((aligned(1024))) char lds_raw[4 * 32768];
    lds_char_t *lds = (lds_char_t *)lds_raw;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // every LDS byte defined before any read (256 bytes per thread)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        f16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (_Float16)(0.001f * (float)((tid + i + e) & 63));
        *(lds_f16x8_t *)(lds + (i * 512 + tid) * 16) = v;
    }
    __syncthreads();
    // buffer resource over [src, src + src_bytes): reads past it return zero
    const uint64_t b = (uint64_t)(uintptr_t)src;
    i32x4 rsrc;
    rsrc[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    rsrc[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32) & 0xffff);
    rsrc[2] = (int)src_bytes;
    rsrc[3] = 0x00020000;
    f32x16 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
    // two fragment sets: a slab's MFMAs take one while its reads fill the other
    f16x8 fa[8], fb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            fa[i][e] = (_Float16)(lane * 0.001f + (i + e) * 0.01f - 0.05f);
            fb[i][e] = fa[i][e];
        }
    i32x4 rsum = {0, 0, 0, 0};
    const uint32_t group_bytes = 256u * pitch;
    const uint32_t ngroups = src_bytes / group_bytes;    // groups of 256 rows src holds
    const uint32_t ncols = pitch / 128u;                 // 128-byte columns of a row
    const uint32_t gstep = (8u * (uint32_t)windows) % ngroups;   // groups the XCDs move on by
    // this workgroup's group and column at slab 0
    uint32_t grp = __builtin_amdgcn_readfirstlane(
        (int)(((blockIdx.x & 7u) * (uint32_t)windows + (blockIdx.x >> 3) % (uint32_t)windows) % ngroups));
    uint32_t col = 0;
    // lane's byte in a 1 KB piece: row lane / 8 of the piece's 8, 16 bytes of
    // 128; with SWIZZLE the chunk of the GEMM's layout: piece `slot` holds
    // rows 8 * slot .. +8, so (row / 2) % 8 = 4 * (slot % 2) + lane / 16
    const uint32_t lane_off = (uint32_t)(lane >> 3) * pitch + (uint32_t)(lane & 7) * 16u;
    const uint32_t lane_off_odd = SWIZZLE
        ? (uint32_t)(lane >> 3) * pitch + (uint32_t)((lane & 7) ^ (4 | (lane >> 4))) * 16u : lane_off;
    const uint32_t lane_off_even = SWIZZLE
        ? (uint32_t)(lane >> 3) * pitch + (uint32_t)((lane & 7) ^ (lane >> 4)) * 16u : lane_off;
    // PANELS: this workgroup's tile of the T x T grid, in the order the GEMM
    // kernels deal tiles to XCDs, and the byte offsets of its A and B panels
    uint32_t pa = 0, pb = 0;
    if constexpr (PANELS) {
        const uint32_t T = src_bytes / (256u * pitch);      // tiles per side
        const int nwg = (int)(T * T), bid = (int)blockIdx.x;
        const int xcd = bid & 7, local = bid >> 3, per = nwg >> 3, rem = nwg & 7;
        const int logical = xcd * per + (xcd < rem ? xcd : rem) + local;
        const int gm = windows, gsz = gm * (int)T;
        const int g = logical / gsz, first_m = g * gm;
        const int rows = ((int)T - first_m) < gm ? ((int)T - first_m) : gm;
        const int in_g = logical - g * gsz;
        const uint32_t tm = (uint32_t)(first_m + in_g % rows), tn = (uint32_t)(in_g / rows);
        pa = __builtin_amdgcn_readfirstlane((int)(tm * 128u * pitch));
        pb = __builtin_amdgcn_readfirstlane((int)((T + tn) * 128u * pitch));
    }
    auto slab = [&](int it, f16x8 (&use)[8], f16x8 (&fill)[8]) {
        if constexpr (LOADS) {
            // vmcnt <= 8: this wave's loads of three slabs ago have landed
            // (vmcnt <= 4: of two slabs ago)
            if constexpr (DEPTH1) __builtin_amdgcn_s_waitcnt((4 & 15) | (7 << 4) | (15 << 8));
            else __builtin_amdgcn_s_waitcnt((8 & 15) | (7 << 4) | (15 << 8));
        }
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        const int stage = (it & 3) * 32768;
        const int rstage = ((it + 2) & 3) * 32768;      // loaded two slabs ago
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            if constexpr (LOADS) {
                if (m % 2 == 0) {
                    const int slot = (m / 2) * 8 + wave;          // 1 KB piece of the 32 KB slab
                    const unsigned dst = (unsigned)(uintptr_t)(lds + stage + slot * 1024);
                    const uint32_t lo = (slot & 1) ? lane_off_odd : lane_off_even;
                    uint32_t voff;
                    if constexpr (PANELS)
                        voff = (slot < 16 ? pa + (uint32_t)slot * 8u * pitch : pb + (uint32_t)(slot - 16) * 8u * pitch)
                               + col * 128u + lo;
                    else
                        voff = grp * group_bytes + (uint32_t)slot * 8u * pitch + col * 128u + lo;
                    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                                 :
                                 : "v"(voff), "s"(rsrc), "{m0}"(__builtin_amdgcn_readfirstlane(dst))
                                 : "memory");
                }
            }
            if constexpr (READS) {
                const int piece = (wave * 8 + m) & 31;        // 1 KB piece of the 32 KB stage
                fill[m] = *(const lds_f16x8_t *)(lds + rstage + piece * 1024 + lane * 16);
            }
            if constexpr (MFMA) {
                // k step t = m / 4, block (i, j) = ((m / 2) % 2, m % 2)
                const int t = m / 4, i = (m / 2) % 2, j = m % 2;
                acc[2 * i + j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(use[2 * t + i], use[4 + 2 * t + j],
                                                                        acc[2 * i + j], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);             // keep the order as written
        }
        if constexpr (READS && !MFMA) {
            // every byte read feeds the result (else the reads would narrow)
#pragma unroll
            for (int i = 0; i < 8; ++i) rsum ^= __builtin_bit_cast(i32x4, fill[i]);
        }
        if (++col == ncols) {
            col = 0;
            if constexpr (!PANELS) grp = grp + gstep >= ngroups ? grp + gstep - ngroups : grp + gstep;
        }
    };
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t w0 = __builtin_amdgcn_s_memrealtime();
    int it = 0;
    for (; it + 1 < iters; it += 2) {
        slab(it, fa, fb);
        slab(it + 1, fb, fa);
    }
    if (it < iters) slab(it, fa, fb);
    if constexpr (LOADS) __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));    // vmcnt(0)
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t w1 = __builtin_amdgcn_s_memrealtime();
    float s = (float)(rsum[0] ^ rsum[1] ^ rsum[2] ^ rsum[3]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[i][r];
    sink[(int64_t)blockIdx.x * 512 + tid] = s;
    if (tid == 0) {
        clocks[2 * (int64_t)blockIdx.x] = t1 - t0;
        clocks[2 * (int64_t)blockIdx.x + 1] = w1 - w0;
    }
}

int hip_status(hipError_t e)
{
    if (e == hipSuccess) return 0;
    g_last_hip_error = (int)e;
    return -200;
}

}  // namespace

extern "C" {

int dgp_mfma_peak(int kind, int64_t workgroups, int32_t iters, float *sink, uint64_t *clocks,
                  void *stream)
{
    if (kind != DGP_MFMA_F32 && kind != DGP_MFMA_F16 && kind != DGP_MFMA_F16_RANDOM) return -1;
    if (workgroups < 1 || workgroups > 65536) return -2;
    if (iters < 1 || iters > (1 << 24)) return -3;
    if (!sink) return -4;
    if (!clocks) return -5;
    hipStream_t s = (hipStream_t)stream;
    const dim3 grid((unsigned)workgroups), block(kThreads);
    if (kind == DGP_MFMA_F16)
        hipLaunchKernelGGL(mfma_peak_kernel<DGP_MFMA_F16>, grid, block, 0, s, (int)iters, sink, clocks);
    else if (kind == DGP_MFMA_F16_RANDOM)
        hipLaunchKernelGGL(mfma_peak_kernel<DGP_MFMA_F16_RANDOM>, grid, block, 0, s, (int)iters, sink, clocks);
    else
        hipLaunchKernelGGL(mfma_peak_kernel<DGP_MFMA_F32>, grid, block, 0, s, (int)iters, sink, clocks);
    return hip_status(hipGetLastError());
}

double dgp_mfma_flops(int kind, int64_t workgroups, int32_t iters)
{
    const double per = (kind == DGP_MFMA_F16 || kind == DGP_MFMA_F16_RANDOM) ? 2.0 * 32 * 32 * 16
                       : kind == DGP_MFMA_F32                                 ? 2.0 * 32 * 32 * 2
                                                                              : 0.0;
    return per * 8.0 * (double)iters * (double)(kThreads / 64) * (double)workgroups;
}

int dgp_copy(const void *src, void *dst, int64_t bytes, void *stream)
{
    if (!src || ((uintptr_t)src & 15)) return -1;
    if (!dst || ((uintptr_t)dst & 15)) return -2;
    if (bytes < 0 || (bytes & 15)) return -3;
    const int64_t n16 = bytes / 16;
    if (n16 == 0) return 0;
    int64_t blocks = (n16 + kThreads - 1) / kThreads;
    if (blocks > 256 * 32) blocks = 256 * 32;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream,
                       (const i32x4 *)src, (i32x4 *)dst, n16);
    return hip_status(hipGetLastError());
}

int dgp_slab_probe(int mode, int64_t workgroups, int32_t iters, int32_t windows, int32_t pitch,
                   const void *src, int64_t src_bytes, float *sink, uint64_t *clocks, void *stream)
{
    if (mode < 1 || mode > 63 || (mode & 7) == 0) return -1;
    if (workgroups < 1 || workgroups > 65536) return -2;
    if (iters < 1 || iters > (1 << 20)) return -3;
    if (windows < 1 || windows > 32) return -4;
    if (pitch < 128 || pitch > 65536 || pitch % 128 != 0) return -5;
    if (!src || ((uintptr_t)src & 15)) return -6;
    if (src_bytes < 256 * (int64_t)pitch || src_bytes % (256 * (int64_t)pitch) != 0 ||
        src_bytes >= ((int64_t)1 << 31))
        return -7;
    if (mode & DGP_SLAB_PANELS) {
        // a T x T tile grid: src holds A and B, T * 128 rows each
        const int64_t T = src_bytes / (256 * (int64_t)pitch);
        if (T * T != workgroups) return -2;
        if (windows > T) return -4;
    }
    if (!sink) return -8;
    if (!clocks) return -9;
    hipStream_t s = (hipStream_t)stream;
    const dim3 grid((unsigned)workgroups), block(512);
    const char *p = (const char *)src;
    const uint32_t nb = (uint32_t)src_bytes;
    switch (mode) {
    case 1: hipLaunchKernelGGL(slab_probe_kernel<1>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 2: hipLaunchKernelGGL(slab_probe_kernel<2>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 3: hipLaunchKernelGGL(slab_probe_kernel<3>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 4: hipLaunchKernelGGL(slab_probe_kernel<4>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 5: hipLaunchKernelGGL(slab_probe_kernel<5>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 6: hipLaunchKernelGGL(slab_probe_kernel<6>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 7: hipLaunchKernelGGL(slab_probe_kernel<7>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 8: hipLaunchKernelGGL(slab_probe_kernel<8>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 9: hipLaunchKernelGGL(slab_probe_kernel<9>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 10: hipLaunchKernelGGL(slab_probe_kernel<10>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 11: hipLaunchKernelGGL(slab_probe_kernel<11>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 12: hipLaunchKernelGGL(slab_probe_kernel<12>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 13: hipLaunchKernelGGL(slab_probe_kernel<13>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 14: hipLaunchKernelGGL(slab_probe_kernel<14>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 15: hipLaunchKernelGGL(slab_probe_kernel<15>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 16: hipLaunchKernelGGL(slab_probe_kernel<16>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 17: hipLaunchKernelGGL(slab_probe_kernel<17>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 18: hipLaunchKernelGGL(slab_probe_kernel<18>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 19: hipLaunchKernelGGL(slab_probe_kernel<19>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 20: hipLaunchKernelGGL(slab_probe_kernel<20>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 21: hipLaunchKernelGGL(slab_probe_kernel<21>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 22: hipLaunchKernelGGL(slab_probe_kernel<22>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 23: hipLaunchKernelGGL(slab_probe_kernel<23>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 24: hipLaunchKernelGGL(slab_probe_kernel<24>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 25: hipLaunchKernelGGL(slab_probe_kernel<25>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 26: hipLaunchKernelGGL(slab_probe_kernel<26>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 27: hipLaunchKernelGGL(slab_probe_kernel<27>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 28: hipLaunchKernelGGL(slab_probe_kernel<28>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 29: hipLaunchKernelGGL(slab_probe_kernel<29>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 30: hipLaunchKernelGGL(slab_probe_kernel<30>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 31: hipLaunchKernelGGL(slab_probe_kernel<31>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 32: hipLaunchKernelGGL(slab_probe_kernel<32>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 33: hipLaunchKernelGGL(slab_probe_kernel<33>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 34: hipLaunchKernelGGL(slab_probe_kernel<34>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 35: hipLaunchKernelGGL(slab_probe_kernel<35>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 36: hipLaunchKernelGGL(slab_probe_kernel<36>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 37: hipLaunchKernelGGL(slab_probe_kernel<37>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 38: hipLaunchKernelGGL(slab_probe_kernel<38>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 39: hipLaunchKernelGGL(slab_probe_kernel<39>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 40: hipLaunchKernelGGL(slab_probe_kernel<40>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 41: hipLaunchKernelGGL(slab_probe_kernel<41>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 42: hipLaunchKernelGGL(slab_probe_kernel<42>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 43: hipLaunchKernelGGL(slab_probe_kernel<43>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 44: hipLaunchKernelGGL(slab_probe_kernel<44>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 45: hipLaunchKernelGGL(slab_probe_kernel<45>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 46: hipLaunchKernelGGL(slab_probe_kernel<46>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 47: hipLaunchKernelGGL(slab_probe_kernel<47>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 48: hipLaunchKernelGGL(slab_probe_kernel<48>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 49: hipLaunchKernelGGL(slab_probe_kernel<49>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 50: hipLaunchKernelGGL(slab_probe_kernel<50>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 51: hipLaunchKernelGGL(slab_probe_kernel<51>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 52: hipLaunchKernelGGL(slab_probe_kernel<52>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 53: hipLaunchKernelGGL(slab_probe_kernel<53>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 54: hipLaunchKernelGGL(slab_probe_kernel<54>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 55: hipLaunchKernelGGL(slab_probe_kernel<55>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 56: hipLaunchKernelGGL(slab_probe_kernel<56>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 57: hipLaunchKernelGGL(slab_probe_kernel<57>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 58: hipLaunchKernelGGL(slab_probe_kernel<58>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 59: hipLaunchKernelGGL(slab_probe_kernel<59>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 60: hipLaunchKernelGGL(slab_probe_kernel<60>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 61: hipLaunchKernelGGL(slab_probe_kernel<61>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    case 62: hipLaunchKernelGGL(slab_probe_kernel<62>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    default: hipLaunchKernelGGL(slab_probe_kernel<63>, grid, block, 0, s, p, nb, (int)iters, (int)windows, (uint32_t)pitch, sink, clocks); break;
    }
    return hip_status(hipGetLastError());
}

int dgp_wall_clock_khz(void)
{
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
    return khz;
}

int dgp_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
