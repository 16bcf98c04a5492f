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
 *   dgp_copy       a plain device copy: sustained HBM read + write rate;
 *   dgp_slab_probe the per-slab work of the fp16 GEMM's 128x128 tile (direct
 *                  loads into LDS, fragment reads from LDS, MFMAs) in any
 *                  combination, which separates the costs of the parts.
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
    DGP_MFMA_F32 = 0,        /* v_mfma_f32_32x32x2_f32: 4096 flops per wave instruction */
    DGP_MFMA_F16 = 1,        /* v_mfma_f32_32x32x16_f16: 32768 flops per wave instruction */
    DGP_MFMA_F16_RANDOM = 2  /* the same on pseudo-random operands in [-1, 1) that change
                                every instruction (the matrix cores' power on real data) */
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

enum {                  /* parts of a slab, combined with | */
    DGP_SLAB_LOADS = 1, /* each wave: 4 direct loads of 1 KB into LDS */
    DGP_SLAB_MFMA = 2,  /* each wave: 8 v_mfma_f32_32x32x16_f16 */
    DGP_SLAB_READS = 4, /* each wave: 8 fragment reads of 1 KB (ds_read_b128) */
    DGP_SLAB_DEPTH1 = 8, /* at each slab's start at most one slab of this wave's
                            loads in flight (else two) */
    DGP_SLAB_PANELS = 16, /* loads of a GEMM tile's A and B panels (see below) */
    DGP_SLAB_SWIZZLE = 32 /* a row's chunks fetched in the fp16 GEMM's lane order */
};

/*
 * Slab probe.  Launches `workgroups` workgroups of 512 threads (8 waves, 128
 * KB of LDS: one per compute unit) that each run `iters` slabs of the fp16
 * GEMM's 128x128 tile without its data flow: per slab a wait until at most
 * two slabs' loads are in flight (one with DGP_SLAB_DEPTH1) and a barrier,
 * then the parts `mode` names (a | of DGP_SLAB_* with at least one of
 * LOADS, MFMA, READS): one load before every second MFMA step and one
 * fragment read before every step, as the GEMM spreads them.
 *
 * The loads (buffer_load_dwordx4 ... lds) see src as rows of `pitch` bytes
 * in groups of 256 rows.  Each slab a workgroup loads one 128-byte column of
 * its group (32 KB), the next column the next slab, as a GEMM tile walks K
 * along its A and B panels (pitch = the operands' row stride).  Workgroup
 * ids are dealt to the 8 XCDs in turn: the workgroups of one XCD share
 * `windows` groups, the XCDs take different groups, and when the columns
 * wrap every workgroup moves on to groups not used before (modulo the groups
 * src holds).  A src that fits L2 stays resident there; a larger one is
 * fetched from the memory side as a GEMM's panels are.  With
 * DGP_SLAB_PANELS the loads are exactly those of a tile of the k-contiguous
 * (nt) GEMM: src holds A and then B, T * 128 rows of `pitch` bytes each,
 * workgroups must be T * T, and workgroup w loads the A and B panels of
 * tile w in the order the GEMM kernels deal tiles to the XCDs, with
 * `windows` (at most T) tile rows per group; one 128-byte column of each
 * panel per slab, the columns wrapping at the end of the rows.  With
 * DGP_SLAB_SWIZZLE the 8 lanes that load one 128-byte row take its 16-byte
 * chunks in the XOR order of the fp16 GEMM's k-contiguous LDS layout (the
 * lane at chunk slot p of row r: chunk p ^ ((r / 2) % 8), r counted within
 * the 256-row window or the 128-row panel) instead of address order.  The reads take the
 * stage loaded two slabs earlier and, with MFMA, are the next slab's
 * operands.
 *   windows 1 .. 32
 *   pitch   128 .. 65536, a multiple of 128 (128: contiguous windows)
 *   src     device, src_bytes readable bytes, 16-byte aligned; src_bytes a
 *           positive multiple of 256 * pitch, below 2^31
 *   sink    device, workgroups * 512 floats, written
 *   clocks  device, workgroups * 2 uint64 values, written: for each
 *           workgroup, the shader-clock ticks (s_memtime) and the constant
 *           wall-clock ticks (s_memrealtime, dgp_wall_clock_khz() per ms)
 *           its first wave spent in the loop
 * Errors: -1 mode invalid, -2 workgroups outside [1, 65536] (with PANELS:
 * not T * T), -3 iters outside [1, 1 << 20], -4 windows outside [1, 32]
 * (with PANELS: above T), -5 pitch invalid, -6 src null or not 16-byte
 * aligned, -7 src_bytes invalid, -8 / -9 null buffers.
 */
int dgp_slab_probe(int mode, int64_t workgroups, int32_t iters, int32_t windows, int32_t pitch,
                   const void *src, int64_t src_bytes, float *sink, uint64_t *clocks, void *stream);

/* Frequency of the s_memrealtime counter of the current device, kHz (0 if unknown). */
int dgp_wall_clock_khz(void);

/* The hipError_t of the last failed HIP call of this library in this thread. */
int dgp_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DENSE_GEMM_PROBE_H */
