// Control probes of the GEMM measurements (libdense_gemm_probe.so): the
// matrix-core peak with the shader clock under load, and a plain device copy.
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

thread_local int g_last_hip_error = 0;

constexpr int kThreads = 256;

// Each wave: `iters` rounds of 8 independent MFMAs (two waves per SIMD when
// two workgroups share a CU keep the matrix core busy).  The first wave of
// each workgroup stamps the loop with the shader clock (s_memtime) and the
// constant wall clock (s_memrealtime).
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
    if constexpr (KIND == DGP_MFMA_F16) {
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
    if (kind != DGP_MFMA_F32 && kind != DGP_MFMA_F16) return -1;
    if (workgroups < 1 || workgroups > 65536) return -2;
    if (iters < 1 || iters > (1 << 24)) return -3;
    if (!sink) return -4;
    if (!clocks) return -5;
    hipStream_t s = (hipStream_t)stream;
    const dim3 grid((unsigned)workgroups), block(kThreads);
    if (kind == DGP_MFMA_F16)
        hipLaunchKernelGGL(mfma_peak_kernel<DGP_MFMA_F16>, grid, block, 0, s, (int)iters, sink, clocks);
    else
        hipLaunchKernelGGL(mfma_peak_kernel<DGP_MFMA_F32>, grid, block, 0, s, (int)iters, sink, clocks);
    return hip_status(hipGetLastError());
}

double dgp_mfma_flops(int kind, int64_t workgroups, int32_t iters)
{
    const double per = kind == DGP_MFMA_F16 ? 2.0 * 32 * 32 * 16 : kind == DGP_MFMA_F32 ? 2.0 * 32 * 32 * 2 : 0.0;
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

int dgp_wall_clock_khz(void)
{
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
    return khz;
}

int dgp_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
