/*
 * dense_gemm_probe.h -- C ABI of libdense_gemm_probe.so: the control probes
 * of the GEMM measurements on AMD Instinct MI355X (gfx950).
 *
 * "Metal GEMM Kernels for LoRA Training on Apple Silicon", section 9 ("What
 * is not measured"), asks for a control benchmark with a known reference,
 * run beside the figures, and for the figures to be rejected when the control
 * lands more than 10% away from its reference (the machine is then busy,
 * throttled or otherwise not the one being characterised).  Two controls are
 * provided, each a kernel whose ideal cost is known exactly:
 *
 *   dgp_mfma_peak  back-to-back independent matrix-core instructions (no
 *                  memory traffic): sustained MFMA rate of the part, and the
 *                  shader clock while it runs;
 *   dgp_copy       a plain device copy: sustained HBM read + write rate.
 *
 * Every function enqueues on `stream` (a hipStream_t, NULL for the default
 * stream), returns after enqueueing, and allocates nothing.  Buffers are
 * device memory owned by the caller.
 *
 * Status: 0 on success; -i when argument i (1-based) is invalid (nothing is
 * enqueued); -200 when a HIP call failed (dgp_last_hip_error() gives the
 * hipError_t).
 */
#ifndef DENSE_GEMM_PROBE_H
#define DENSE_GEMM_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    DGP_MFMA_F32 = 0,   /* v_mfma_f32_32x32x2_f32: 4096 flops per wave instruction */
    DGP_MFMA_F16 = 1    /* v_mfma_f32_32x32x16_f16: 32768 flops per wave instruction */
};

/*
 * Matrix-core peak probe.  Launches `workgroups` workgroups of 256 threads
 * (4 waves); every wave runs `iters` rounds of 8 independent MFMAs of the
 * given kind on register operands.
 *   sink    device, workgroups * 256 floats, written (keeps the results live)
 *   clocks  device, workgroups * 2 uint64 values, written: for each
 *           workgroup, the shader-clock ticks (s_memtime) and the constant
 *           wall-clock ticks (s_memrealtime, dgp_wall_clock_khz() per ms)
 *           that its first wave spent in the loop; their ratio is the shader
 *           clock under matrix-core load
 * Errors: -1 kind unknown, -2 workgroups outside [1, 65536], -3 iters
 * outside [1, 1 << 24], -4 / -5 null buffers.
 */
int dgp_mfma_peak(int kind, int64_t workgroups, int32_t iters, float *sink, uint64_t *clocks,
                  void *stream);

/* Matrix-core flops one dgp_mfma_peak launch performs (0 for an unknown kind). */
double dgp_mfma_flops(int kind, int64_t workgroups, int32_t iters);

/*
 * Device copy dst[0, bytes) = src[0, bytes) with 16-byte loads and stores
 * (grid-stride loop), for the HBM control: it moves exactly 2 * bytes.
 * Errors: -1 / -2 null or not 16-byte aligned, -3 bytes negative or not a
 * multiple of 16.  The ranges must not overlap.
 */
int dgp_copy(const void *src, void *dst, int64_t bytes, void *stream);

/* Frequency of the s_memrealtime counter of the current device, kHz (0 if unknown). */
int dgp_wall_clock_khz(void);

/* The hipError_t of the last failed HIP call of this library in this thread. */
int dgp_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DENSE_GEMM_PROBE_H */
