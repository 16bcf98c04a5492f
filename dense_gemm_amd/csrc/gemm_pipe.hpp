// GEMM for gfx950 with a multi-stage LDS ring fed by direct global->LDS
// loads, for 16-bit operands (fp16 or bf16, fp32 accumulation) and for fp32.
//
//   C[BM x BN tile] = act(alpha * sum_k op(A)[rows, k] op(B)[k, cols]
//                         + beta * C + bias[cols]),
//   fp16 / bf16: v_mfma_f32_32x32x16_f16 / _bf16 with fp32 accumulators
//   ("Metal GEMM Kernels for LoRA Training on Apple Silicon", section 1: the
//   fp32 accumulator keeps the fast path), K slabs of 64;
//   fp32: v_mfma_f32_32x32x2_f32, K slabs of 16 (32 on one 64 x 64 kernel).
//   The bias and activation are the fused epilogue of "From a C loop to a GPU
//   kernel", "Fusion"; grid y is the batch of a strided-batched call (the
//   per-head offsets of "Metal GEMM Kernels for LoRA Training", section 8).
//
// Why a different kernel from gemm_mfma.hpp: at 2048^3 one 128 x 128 tile per
// compute unit leaves a single wave per SIMD, and one 64-wide K slab is only
// ~512 MFMA cycles, shorter than a load round trip.  So the slabs are
// prefetched STAGES-1 deep, and the loads go straight to LDS
// (buffer_load_dwordx4 ... lds: each lane's 16 bytes land at M0 + 16*lane),
// which costs no registers and no transposing VALU work.  The buffer form
// addresses each lane with a 32-bit offset from a wave-uniform base held in
// scalar registers; beside the MFMAs it measured about half the matrix-core
// stall of the global form, whose 64-bit per-lane addresses the SIMD sends
// to the address unit (a microbenchmark of one GEMM slab per iteration: 615
// cycles against 720, with 475 for the MFMAs alone and 500 for the loads).
//
// fp16 LDS layouts (both conflict-free for the fragment reads):
//   k-contiguous operand (A not transposed, B transposed): [BMN][64] halfs,
//     128-byte rows; the 16-byte chunk c of row r sits at chunk c ^ ((r>>1)&7),
//     so the 16 rows read together by a quarter wave hit 16 distinct bank
//     groups.  Fragments: one ds_read_b128 = 8 consecutive k of one row.
//   m/n-contiguous operand (A transposed, B not transposed): [64][BMN]
//     halfs, rows of BMN*2 bytes; the 64-byte quad q of row k sits at quad
//     q ^ swz(k): k&3 when a row has 4 or more quads (BMN >= 128), (k>>1)&1
//     when it has 2 (BMN = 64: rows 128 bytes = 32 banks apart, so rows k
//     and k+2 would meet), none for BMN = 32 (64-byte rows already fall on
//     distinct banks for the 4 rows a read takes).  Fragments come from
//     ds_read_b64_tr_b16, the hardware
//     transposing read: in each 16-lane group, lanes 4t..4t+3 name row t of a
//     4 x 16 block and lane j receives column j, i.e. 4 consecutive k of its
//     own m (or n) -- the MFMA operand layout -- with no write-side transpose
//     (the page's section 3 transposes on the write; gfx950 can do it on the
//     read).
// fp32 LDS layouts, K slab BK = 16 or 32: k-contiguous operand [BMN][BK]
// floats, rows of 64 or 128 bytes, the 16-byte chunk c of row r at chunk
// c ^ ((r>>2)&3) (BK = 16) or c ^ (r&7) ^ ((r>>3)&1) (BK = 32); one
// ds_read_b128 gives a lane 4 consecutive k (4 MFMA steps).  m/n-contiguous
// operand [BK][BMN] floats, the 128-byte chunk q of row k at
// q ^ ((k/(BK/2))&1); a lane reads one float per MFMA step, the two
// half-waves from rows k and k+BK/2 (different bank halves after the
// swizzle).  In both types lane half h of MFMA step s takes k = h*BK/2 + s,
// the same for both operands.
// The swizzle is applied by choosing which global address each lane fetches,
// since a direct load writes its lanes contiguously.
//
// Pipeline per K slab kt (one barrier per slab), 16-bit tiles up to 256 x 128:
//   wait for this thread's loads of slab kt+1; barrier (slab kt+1 visible to
//   all, and every wave holds its fragments of slab kt in registers); issue
//   the loads of a later slab into a stage whose fragments every wave has
//   read; read the fragments of slab kt+1 into the second register set while
//   the MFMAs of slab kt run.  16-bit 256 x 256 tiles (whose accumulators
//   leave registers for one k step's fragments, not a slab's): the barrier
//   sits before each slab's last k step, which overlaps the next slab's first
//   fragment reads (see the loop).  fp32 (whose larger wave tiles leave no
//   registers for a second fragment set): wait for slab kt; barrier; issue
//   slab kt+STAGES-1 into the stage of slab kt-1; fragment reads and MFMAs
//   of slab kt.  (For fp32, moving the barrier into the middle of a slab
//   measured slower: it drains the MFMA queue mid-slab.)
//
// Host-side preconditions (checked by the dispatcher): 16-byte loads (LB =
// 16) need A and B 16-byte aligned with lda, ldb multiples of 16 bytes and
// the m/n-contiguous operand's extent (M if A is transposed, N if B is not) a
// multiple of 16 bytes; 4-byte loads (LB = 4) need 4-byte alignment, and for
// 16-bit operands even strides and an even m/n-contiguous extent.  256 rows
// of each stored operand must span less than 2^31 bytes (32-bit offsets).  A
// last slab shorter than BK is loaded through registers with zero fill.  Rows
// or columns past M or N are fetched from a clamped, valid address; they only
// feed outputs that the guarded epilogue never stores.
#pragma once

#include <type_traits>

#include "gemm_common.hpp"

namespace dg {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) char lds_char_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

constexpr int PIPE_BK = 64;

// Buffer resource of a raw byte buffer at `base` (gfx9 layout: 48-bit base,
// stride 0, num_records, format dword).  num_records is the largest value:
// the kernels bound every offset themselves (rows clamped to the matrix), as
// the global form did.  The fields are made wave-uniform so that the
// resource lives in scalar registers, as the instruction requires.
typedef int i32x4_rsrc __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_rsrc buffer_rsrc(const char *base)
{
    const uint64_t b = (uint64_t)(uintptr_t)base;
    i32x4_rsrc r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32) & 0xffff);
    r[2] = -1;
    r[3] = 0x00020000;
    return r;
}

// One direct load: 16 bytes per lane from base + voff into LDS at
// lds_addr + 16 * lane.  Inline asm, so that the compiler does not track it:
// it would otherwise wait for every direct load in flight (all prefetched
// slabs) before each LDS read and barrier.  Completion is awaited explicitly
// with wait_vmcnt (vector-memory loads retire in order).  M0 holds the
// wave-uniform LDS destination.
__device__ __forceinline__ void load_lds16(uint32_t voff, i32x4_rsrc rsrc, unsigned lds_addr)
{
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr))
                 : "memory");
}

// The 4-byte form (operands whose rows are not 16-byte aligned): lane l's 4
// bytes land at lds_addr + 4 * l.
__device__ __forceinline__ void load_lds4(uint32_t voff, i32x4_rsrc rsrc, unsigned lds_addr)
{
    asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr))
                 : "memory");
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// One 16-bit operand (fp16 or bf16) of the pipelined kernel (K slab 64).
//   KCONT: stored [ext][K] (k contiguous); else stored [K][ext].
//   LB: bytes per lane per direct load: 16, or 4 (two elements) for rows
//   that are 4-byte but not 16-byte aligned.  The LDS layout is the same;
//   each lane fetches the element pair that belongs at its LDS slot.
template <typename E, int BMN, bool KCONT, int NW, int LB = 16>
struct PipeOperandH {
    static_assert(LB == 16 || LB == 4, "16- or 4-byte direct loads");
    typedef E V8 __attribute__((ext_vector_type(8)));
    typedef E V2 __attribute__((ext_vector_type(2)));
    typedef __attribute__((address_space(3))) V8 lds_v8_t;
    typedef __attribute__((address_space(3))) V2 lds_v2_t;
    static constexpr int BK = PIPE_BK;
    static constexpr int BYTES = BMN * PIPE_BK * 2;      // one stage
    static constexpr int SPAN = 64 * LB;                  // LDS bytes of one wave-wide load
    static constexpr int LOADS = BYTES / (NW * SPAN);     // loads per thread per slab
    static_assert(LOADS * NW * SPAN == BYTES, "slab must split into whole loads");
    static constexpr int ROW_BYTES = KCONT ? PIPE_BK * 2 : BMN * 2;
    static constexpr int ROWS_PER_LOAD = 1024 / ROW_BYTES;  // rows one wave-wide load fills
    static constexpr int QUADS = ROW_BYTES / 64;             // 64-byte quads per row (m/n-contiguous)
    static_assert(KCONT || BMN == 32 || BMN == 64 || BMN % 128 == 0, "m/n-contiguous tile width");

    // XOR applied to the quad index of row k (m/n-contiguous layout)
    __device__ static __forceinline__ int swz(int k)
    {
        return QUADS >= 4 ? (k & 3) : (QUADS == 2 ? ((k >> 1) & 1) : 0);
    }

    const char *base;            // the current slab's tile origin (wave-uniform)
    uint32_t off[LOADS];         // per-lane byte offsets from base
    int64_t step;                // bytes to advance per slab

    // Per-lane offsets for the slab at k = 0.  mn0: first row (m or n) of
    // the tile; ext: M or N; ld: row stride of the stored matrix.  Offsets
    // stay below 256 * ld * 2 bytes (the dispatcher keeps that under 2^31).
    __device__ __forceinline__ void init(const E *g, int64_t ld, int mn0, int ext, int wave,
                                         int lane)
    {
        base = (const char *)(KCONT ? g + (int64_t)mn0 * ld : g + mn0);
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            if constexpr (LB == 16) {
                const int rbase = (i * NW + wave) * ROWS_PER_LOAD;  // first LDS row of this load
                if constexpr (KCONT) {
                    const int r = rbase + (lane >> 3);
                    const int c = (lane & 7) ^ ((r >> 1) & 7);      // logical 16-byte chunk (8 k)
                    int row = mn0 + r;
                    row = row < ext ? row : ext - 1;
                    off[i] = (uint32_t)(((int64_t)(row - mn0) * ld + c * 8) * 2);
                } else {
                    const int r = rbase + (lane / (ROW_BYTES / 16));  // k row
                    const int p = lane % (ROW_BYTES / 16);            // physical 16-byte slot
                    const int q = (p >> 2) ^ swz(r);                  // logical 64-byte quad
                    int col = mn0 + q * 32 + (p & 3) * 8;
                    col = col < ext ? col : ext - 8;
                    off[i] = (uint32_t)(((int64_t)r * ld + (col - mn0)) * 2);
                }
            } else {
                const int b = (i * NW + wave) * SPAN + lane * 4;      // LDS byte in the stage
                const int r = b / ROW_BYTES, w = b % ROW_BYTES;
                const int p = w >> 4, e = (w >> 2) & 3;               // 16-byte slot, element pair
                if constexpr (KCONT) {
                    const int c = p ^ ((r >> 1) & 7);
                    int row = mn0 + r;
                    row = row < ext ? row : ext - 1;
                    off[i] = (uint32_t)(((int64_t)(row - mn0) * ld + c * 8 + 2 * e) * 2);
                } else {
                    const int q = (p >> 2) ^ swz(r);
                    int col = mn0 + q * 32 + (p & 3) * 8 + 2 * e;
                    col = col < ext ? col : ext - 2;                  // ext is even here
                    off[i] = (uint32_t)(((int64_t)r * ld + (col - mn0)) * 2);
                }
            }
        }
        step = (KCONT ? PIPE_BK : PIPE_BK * ld) * 2;
    }

    __device__ __forceinline__ void advance() { base += step; }

    // The last slab when K is not a multiple of 64: the same 16-byte pieces
    // into the same LDS slots, but through registers, with k at or beyond K
    // read as zero.  Happens once per kernel; the wave waits for these loads.
    __device__ __forceinline__ void issue_tail(lds_char_t *lds, int wave, int lane, int krem)
    {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const E *src = (const E *)(base + off[i]);
            if constexpr (LB == 16) {
                lds_char_t *dst = lds + (i * NW + wave) * 1024 + lane * 16;
                int valid;  // halfs of this 16-byte piece that lie before K
                if constexpr (KCONT) {
                    const int r = (i * NW + wave) * ROWS_PER_LOAD + (lane >> 3);
                    const int c = (lane & 7) ^ ((r >> 1) & 7);
                    valid = krem - c * 8;
                } else {
                    const int r = (i * NW + wave) * ROWS_PER_LOAD + (lane / (ROW_BYTES / 16));
                    valid = r < krem ? 8 : 0;
                }
                V8 v;
                if (valid >= 8) {
                    v = *(const V8 *)src;
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        E x = (E)0.f;
                        if (e < valid) x = src[e];
                        v[e] = x;
                    }
                }
                *(lds_v8_t *)dst = v;
            } else {
                const int b = (i * NW + wave) * SPAN + lane * 4;
                const int r = b / ROW_BYTES, w = b % ROW_BYTES;
                const int p = w >> 4, e = (w >> 2) & 3;
                // halfs of this pair that lie before K
                const int valid = KCONT ? krem - ((p ^ ((r >> 1) & 7)) * 8 + 2 * e) : (r < krem ? 2 : 0);
                V2 v;
                v[0] = valid >= 1 ? src[0] : (E)0.f;
                v[1] = valid >= 2 ? src[1] : (E)0.f;
                *(lds_v2_t *)(lds + b) = v;
            }
        }
        advance();
    }

    // Issue this slab's direct loads into the stage at `lds` and advance.
    __device__ __forceinline__ void issue(lds_char_t *lds, int wave)
    {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) issue_one(lds, wave, i);
        advance();
    }

    // Load i of this slab alone (the main loop spreads a slab's loads
    // between its MFMAs and calls advance() after the last one).
    __device__ __forceinline__ void issue_one(lds_char_t *lds, int wave, int i)
    {
        const unsigned dst = (unsigned)(uintptr_t)(lds + (i * NW + wave) * SPAN);
        if constexpr (LB == 16) load_lds16(off[i], buffer_rsrc(base), dst);
        else load_lds4(off[i], buffer_rsrc(base), dst);
    }

    // MFMA operand of block rows [b0, b0+32) for k-step kk (16 k) of a stage.
    __device__ __forceinline__ V8 frag(const lds_char_t *lds, int b0, int kk, int lane) const
    {
        if constexpr (KCONT) {
            const int r = b0 + (lane & 31);
            const int c = 2 * kk + (lane >> 5);
            const int p = c ^ ((r >> 1) & 7);
            return *(const lds_v8_t *)(lds + r * ROW_BYTES + p * 16);
        } else {
            const int g = lane >> 4, j = lane & 15, t = j >> 2, s = j & 3;
            const int q = b0 >> 5;
            const int colb = (16 * (g & 1) + 4 * s) * 2;   // byte offset inside the 64-byte quad
            const int k0 = 16 * kk + 8 * (g >> 1) + t;
            const lds_char_t *p0 = lds + k0 * ROW_BYTES + ((q ^ swz(k0)) << 6) + colb;
            const lds_char_t *p1 = p0 + 4 * ROW_BYTES;      // rows k0 + 4 (same swizzle)
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)p0);
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)p1);
            typedef short i16x8 __attribute__((ext_vector_type(8)));
            const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            return __builtin_bit_cast(V8, v);
        }
    }
};


// One fp32 operand of the pipelined kernel (K slab BKS: 16 or 32).
//   KCONT: stored [ext][K] (k contiguous); else stored [K][ext].
//   LB: bytes per lane per direct load: 16, or 4 for rows that are not
//   16-byte aligned (any fp32 layout).  The LDS layout is the same; a
//   4-byte load fills a quarter of the bytes a 16-byte load does, and each
//   lane fetches the element that belongs at its LDS slot.
//   BKS: a slab of 32 makes each k-contiguous row of a stage one whole
//   128-byte line (64 bytes, half a line, at 16).
template <int BMN, bool KCONT, int NW, int LB = 16, int BKS = 16>
struct PipeOperandS {
    static_assert(LB == 16 || LB == 4, "16- or 4-byte direct loads");
    static_assert(BKS == 16 || BKS == 32, "slabs of 16 or 32 k");
    static constexpr int BK = BKS;
    static constexpr int CH = BK / 4;                      // 16-byte chunks of a k-contiguous row
    static constexpr int CH_LOG = BK == 16 ? 2 : 3;
    static constexpr int HK = BK / 2;                      // k rows read by one half-wave
    static constexpr int HK_LOG = BK == 16 ? 3 : 4;
    // Chunk swizzle of k-contiguous row r.  A fragment read has lane l read
    // row b0 + l%32 at one logical chunk; the swizzle spreads 8 consecutive
    // rows over the 8 chunks of 128 bytes, and 16 consecutive rows over the
    // 16 of 256 bytes (64-byte rows: 4 chunks, by (r >> 2) & 3 beside r & 1;
    // 128-byte rows: 8 chunks, by r & 7, flipped for rows 8-15 of each 16).
    static __device__ __forceinline__ int swz(int r)
    {
        return BK == 16 ? ((r >> 2) & 3) : ((r & 7) ^ ((r >> 3) & 1));
    }
    // Half swap of m/n-contiguous k row r: which 128-byte half of a 64-wide
    // block row holds columns 0-31; the two half-waves (k rows HK apart)
    // then read different halves.
    static __device__ __forceinline__ int hsw(int r) { return (r >> HK_LOG) & 1; }
    // A 32-wide m/n-contiguous tile has 128-byte k rows, one block wide: there
    // the rows of the second half of the slab swap places in pairs (k row r
    // sits at LDS row r ^ 1 when r >= HK), so that the two half-waves of a
    // fragment read, HK rows apart, fall on rows of opposite parity and so on
    // different halves of the 64 banks.
    static constexpr bool NARROW = !KCONT && BMN == 32;
    static __device__ __forceinline__ int krow(int r) { return NARROW ? r ^ ((r >> HK_LOG) & 1) : r; }
    static constexpr int BYTES = BMN * BK * 4;            // one stage
    static constexpr int SPAN = 64 * LB;                   // LDS bytes of one wave-wide load
    static constexpr int LOADS = BYTES / (NW * SPAN);      // loads per thread per slab
    static_assert(LOADS * NW * SPAN == BYTES, "slab must split into whole loads");
    static constexpr int ROW_BYTES = KCONT ? BK * 4 : BMN * 4;
    static constexpr int ROWS_PER_LOAD = 1024 / ROW_BYTES;
    static_assert(ROWS_PER_LOAD >= 1, "rows of at most 1 KiB");

    const char *base;            // the current slab's tile origin (wave-uniform)
    uint32_t off[LOADS];         // per-lane byte offsets from base
    int64_t step;                // bytes to advance per slab

    // The stored element behind LDS byte b of a stage: k row / m-n row r and
    // the element's place; as the 16-bit operand, offsets stay below
    // 256 * ld * 4 bytes.
    __device__ __forceinline__ void init(const float *g, int64_t ld, int mn0, int ext, int wave,
                                         int lane)
    {
        base = (const char *)(KCONT ? g + (int64_t)mn0 * ld : g + mn0);
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            if constexpr (LB == 16) {
                const int rbase = (i * NW + wave) * ROWS_PER_LOAD;
                if constexpr (KCONT) {
                    const int r = rbase + (lane >> CH_LOG);
                    const int c = (lane & (CH - 1)) ^ swz(r);     // logical 16-byte chunk (4 k)
                    int row = mn0 + r;
                    row = row < ext ? row : ext - 1;
                    off[i] = (uint32_t)(((int64_t)(row - mn0) * ld + c * 4) * 4);
                } else {
                    const int r = krow(rbase + (lane / (ROW_BYTES / 16)));  // k row
                    const int p = lane % (ROW_BYTES / 16);            // physical 16-byte slot
                    const int q = NARROW ? 0 : (p >> 3) ^ hsw(r);     // logical 128-byte chunk
                    int col = mn0 + q * 32 + (p & 7) * 4;
                    col = col < ext ? col : ext - 4;
                    off[i] = (uint32_t)(((int64_t)r * ld + (col - mn0)) * 4);
                }
            } else {
                const int b = (i * NW + wave) * SPAN + lane * 4;      // LDS byte in the stage
                const int r = b / ROW_BYTES, w = b % ROW_BYTES;
                const int p = w >> 4, e = (w >> 2) & 3;               // 16-byte slot, element
                if constexpr (KCONT) {
                    const int c = p ^ swz(r);
                    int row = mn0 + r;
                    row = row < ext ? row : ext - 1;
                    off[i] = (uint32_t)(((int64_t)(row - mn0) * ld + c * 4 + e) * 4);
                } else {
                    const int k = krow(r);
                    const int q = NARROW ? 0 : (p >> 3) ^ hsw(k);
                    int col = mn0 + q * 32 + (p & 7) * 4 + e;
                    col = col < ext ? col : ext - 1;
                    off[i] = (uint32_t)(((int64_t)k * ld + (col - mn0)) * 4);
                }
            }
        }
        step = (KCONT ? BK : BK * ld) * 4;
    }

    __device__ __forceinline__ void advance() { base += step; }

    __device__ __forceinline__ void issue_tail(lds_char_t *lds, int wave, int lane, int krem)
    {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const float *src = (const float *)(base + off[i]);
            if constexpr (LB == 16) {
                lds_char_t *dst = lds + (i * NW + wave) * 1024 + lane * 16;
                int valid;  // floats of this 16-byte piece that lie before K
                if constexpr (KCONT) {
                    const int r = (i * NW + wave) * ROWS_PER_LOAD + (lane >> CH_LOG);
                    const int c = (lane & (CH - 1)) ^ swz(r);
                    valid = krem - c * 4;
                } else {
                    const int r = krow((i * NW + wave) * ROWS_PER_LOAD + (lane / (ROW_BYTES / 16)));
                    valid = r < krem ? 4 : 0;
                }
                f32x4 v;
                if (valid >= 4) {
                    v = *(const f32x4 *)src;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float x = 0.f;
                        if (e < valid) x = src[e];
                        v[e] = x;
                    }
                }
                *(__attribute__((address_space(3))) f32x4 *)dst = v;
            } else {
                const int b = (i * NW + wave) * SPAN + lane * 4;
                const int r = b / ROW_BYTES, w = b % ROW_BYTES;
                const int p = w >> 4, e = (w >> 2) & 3;
                const int k = KCONT ? (p ^ swz(r)) * 4 + e : krow(r);   // this element's k
                *(__attribute__((address_space(3))) float *)(lds + b) = k < krem ? *src : 0.f;
            }
        }
        advance();
    }

    __device__ __forceinline__ void issue(lds_char_t *lds, int wave)
    {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) issue_one(lds, wave, i);
        advance();
    }

    // Load i of this slab alone (the main loop spreads a slab's loads
    // between its MFMAs and calls advance() after the last one).
    __device__ __forceinline__ void issue_one(lds_char_t *lds, int wave, int i)
    {
        const unsigned dst = (unsigned)(uintptr_t)(lds + (i * NW + wave) * SPAN);
        if constexpr (LB == 16) load_lds16(off[i], buffer_rsrc(base), dst);
        else load_lds4(off[i], buffer_rsrc(base), dst);
    }

    // The operand values of MFMA steps 4*c2 .. 4*c2+3 for block rows
    // [b0, b0+32): lane l holds row (or column) b0 + l%32 and
    // k = (l/32)*HK + 4*c2 + e, e = 0..3.
    __device__ __forceinline__ f32x4 frag4(const lds_char_t *lds, int b0, int c2, int lane) const
    {
        typedef __attribute__((address_space(3))) f32x4 lds_f32x4_t;
        typedef __attribute__((address_space(3))) float lds_float_t;
        const int h = lane >> 5;
        if constexpr (KCONT) {
            const int r = b0 + (lane & 31);
            const int c = (h << (CH_LOG - 1)) + c2;
            const int p = c ^ swz(r);
            return *(const lds_f32x4_t *)(lds + r * ROW_BYTES + p * 16);
        } else if constexpr (NARROW) {
            // k row HK*h + 4*c2 + e sits at LDS row HK*h + ((4*c2 + e) ^ h)
            const lds_char_t *base = lds + (h << HK_LOG) * ROW_BYTES + (lane & 31) * 4;
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = *(const lds_float_t *)(base + ((4 * c2 + e) ^ h) * ROW_BYTES);
            return v;
        } else {
            const int q = (b0 >> 5) ^ h;   // hsw(k) == h for k = HK*h + ...
            const lds_char_t *base = lds + ((h << HK_LOG) + 4 * c2) * ROW_BYTES + q * 128 + (lane & 31) * 4;
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = *(const lds_float_t *)(base + e * ROW_BYTES);
            return v;
        }
    }
};


// The end of an fp32 kernel with K groups (one 32 x 32 block per wave).
// Wave w = g*NWG + q (group g, sub-tile q) stages its partial block as fp32
// [32][EPI_LD] in LDS slot w; after a barrier, wave w takes rows
// 32/KSPLIT*g .. +32/KSPLIT-1 of sub-tile q, 8 rows per pass (lane l row
// l/8 of the pass, columns 4*(l%8) .. +3), sums the KSPLIT partials in increasing group order,
// and writes alpha*sum + beta*C + bias and the activation (fp32, 16-byte
// stores where the row allows), or the raw sum to the split-K workspace.
template <int KSPLIT, int NWG, int WAVES_N, int WM, int WN, int EPI_LD>
__device__ __forceinline__ void fp32_groups_epilogue(const GemmParams &p, lds_char_t *smem, const f32x16 &acc,
                                                     int wave, int lane, int m0, int n0, int split)
{
    typedef __attribute__((address_space(3))) float lds_float_t;
    typedef __attribute__((address_space(3))) f32x4 lds_f32x4_t;
    constexpr int SLOT = 32 * EPI_LD * 4;
    constexpr int ROWS = 32 / KSPLIT;                // rows of the block per group, 8 per pass
    lds_char_t *stg = smem + wave * SLOT;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + (lane >> 5) * 4 + (r & 3);
        *(lds_float_t *)(stg + (row * EPI_LD + (lane & 31)) * 4) = acc[r];
    }
    __syncthreads();
    const int g = wave / NWG, q = wave % NWG;
    const int lc = (lane & 7) * 4;
    const int gcol = n0 + (q % WAVES_N) * WN + lc;
#pragma unroll
    for (int pass = 0; pass < ROWS / 8; ++pass) {
        const int lr = ROWS * g + 8 * pass + (lane >> 3);
        float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int gg = 0; gg < KSPLIT; ++gg) {
            const f32x4 x = *(const lds_f32x4_t *)(smem + (gg * NWG + q) * SLOT + (lr * EPI_LD + lc) * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] += x[e];
        }
        const int grow = m0 + (q / WAVES_N) * WM + lr;
        if (grow >= p.M) continue;
        if (p.splits > 1) {
            float *w = p.ws + ((int64_t)split * p.M + grow) * p.N + gcol;
            if (gcol + 4 <= p.N && (p.N & 3) == 0) {
                *(f32x4 *)w = (f32x4){v[0], v[1], v[2], v[3]};
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (gcol + e < p.N) w[e] = v[e];
            }
            continue;
        }
        float *c = (float *)p.C + (int64_t)grow * p.ldc + gcol;
        if (p.c_vec && gcol + 4 <= p.N) {
            float cin[4] = {0.f, 0.f, 0.f, 0.f};
            if (p.beta != 0.f) {
                const f32x4 ci = *(const f32x4 *)c;
#pragma unroll
                for (int e = 0; e < 4; ++e) cin[e] = ci[e];
            }
            epilogue_row<float, 4>(p, v, cin, gcol);
            *(f32x4 *)c = (f32x4){v[0], v[1], v[2], v[3]};
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (gcol + e < p.N) {
                    const float cin = p.beta != 0.f ? c[e] : 0.f;
                    c[e] = epilogue_value<float>(p, v[e], cin, gcol + e);
                }
            }
        }
    }
}

// Waves: (BM/WM) x (BN/WN) sub-tiles per K group, KSPLIT groups.  Group g
// runs the 16-k steps [g*4/KSPLIT, (g+1)*4/KSPLIT) of every slab, so with a
// 128 x 128 tile of 64 x 64 sub-tiles and KSPLIT = 2 each SIMD holds two
// waves (one per group): while one waits on LDS or the barrier the other
// keeps the matrix core busy, at unchanged LDS read traffic per MFMA.  At the
// end the two partial accumulators of a sub-tile are summed through LDS: each
// wave keeps half of its blocks and hands the other half to its partner (the
// same sub-tile in the other group).  A 256 x 128 tile gets its two waves per
// SIMD from eight 64 x 64 sub-tiles instead (KSPLIT = 1).
// fp32 K groups (one 32 x 32 block per wave, KSPLIT of 2 or 4): group g runs
// the MFMA steps [g, g+1) * BK/(2*KSPLIT) of every slab, so a 32 x 32 tile
// with four groups puts a wave on each SIMD of its CU; at the end every wave
// stages its partial block in LDS and group g sums rows [g, g+1) * 32/KSPLIT
// of its sub-tile over the groups, in increasing group order.
// LB: bytes per lane of each direct load, 16, or 4 for rows that are not
// 16-byte aligned.  LBMN (default LB): the same for an m/n-contiguous
// operand alone; LB = 16 with LBMN = 4 serves rows that are 4-byte aligned
// only: the k-contiguous operand's 16-byte pieces lie inside its rows (its
// K tail goes through registers) and need no 16-byte alignment, while an
// m/n-contiguous extent that is not a multiple of 4 needs element loads.  TC: the element type of C and the bias (T, or fp32 for an
// fp32 output of 16-bit operands).  FBK: the K slab of fp32 operands, 16 or
// 32 (16-bit operands always take 64).
template <typename T, int BM, int BN, int WM, int WN, bool TA, bool TB, int STAGES, int KSPLIT,
          int LB = 16, typename TC = T, int FBK = 16, int LBMN = LB>
__global__ __launch_bounds__(64 * (BM / WM) * (BN / WN) * KSPLIT, 2) void gemm_pipe_kernel(GemmParams p)
{
    constexpr bool HALF = sizeof(T) == 2;          // fp16 or bf16 operands
    typedef T V8 __attribute__((ext_vector_type(8)));
    constexpr int WAVES_N = BN / WN;
    constexpr int NWG = (BM / WM) * WAVES_N;       // waves per K group
    constexpr int NW = NWG * KSPLIT;               // waves per workgroup
    static_assert(NW == 4 || NW == 8, "4 or 8 waves");
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int NB = TM * TN;                    // 32x32 blocks per wave
    constexpr int KPW = (PIPE_BK / 16) / KSPLIT;   // fp16: 16-k steps per wave per slab
    static_assert(KPW >= 1 && KPW * KSPLIT == PIPE_BK / 16, "K split");
    static_assert(!HALF || KSPLIT == 1 || NB % 2 == 0, "blocks split between partners");
    static_assert(HALF || KSPLIT == 1 || ((KSPLIT == 2 || KSPLIT == 4) && NB == 1 && (FBK / 8) % KSPLIT == 0),
                  "fp32 K groups: one block per wave, whole 4-step fragment groups per group");
    static_assert(FBK == 16 || (!HALF && FBK == 32), "fp32 slabs of 16 or 32");
    // LB: bytes per direct load of a k-contiguous operand; LBMN: of an
    // m/n-contiguous one
    constexpr int LBA = TA ? LBMN : LB, LBB = TB ? LB : LBMN;
    typedef typename std::conditional<HALF, PipeOperandH<T, BM, !TA, NW, LBA>, PipeOperandS<BM, !TA, NW, LBA, FBK>>::type OpA;
    typedef typename std::conditional<HALF, PipeOperandH<T, BN, TB, NW, LBB>, PipeOperandS<BN, TB, NW, LBB, FBK>>::type OpB;
    constexpr int BK = OpA::BK;
    constexpr int STAGE_BYTES = OpA::BYTES + OpB::BYTES;
    constexpr int SMEM = STAGES * STAGE_BYTES;
    constexpr int XCHG_BYTES = NW * (NB / 2) * 4096;     // partner exchange
    constexpr int EPI_LD = 40;                           // floats per staged row (32 + 8)
    constexpr int EPI_BYTES = NW * 32 * EPI_LD * 4;      // epilogue staging, one block per wave
    static_assert(!HALF || KSPLIT == 1 || XCHG_BYTES <= SMEM, "exchange fits the ring");
    static_assert(EPI_BYTES <= SMEM, "epilogue staging fits the ring");
    __shared__ __attribute__((aligned(1024))) char smem_raw[SMEM];
    lds_char_t *smem = (lds_char_t *)smem_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kgroup = wave / NWG;
    const int wq = wave % NWG;
    const int wm0 = (wq / WAVES_N) * WM;
    const int wn0 = (wq % WAVES_N) * WN;
    const int kk0 = kgroup * KPW;
    select_batch<T, TC>(p, blockIdx.y);
    int bid, split, k_begin, Kl;
    split_of(p, bid, split, k_begin, Kl);
    int tm, tn;
    tile_coords(bid, p, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int nk = (Kl + BK - 1) / BK;

    // this split's k range starts at k_begin (a multiple of the slab)
    OpA ga;
    OpB gb;
    ga.init((const T *)p.A + (TA ? (int64_t)k_begin * p.lda : (int64_t)k_begin), p.lda, m0, p.M,
            wave, lane);
    gb.init((const T *)p.B + (TB ? (int64_t)k_begin : (int64_t)k_begin * p.ldb), p.ldb, n0, p.N,
            wave, lane);

    // slab s of nk goes through issue_tail when it is a partial last slab
    const int krem = Kl - (nk - 1) * BK;         // k of the last slab (1..BK)
    auto issue_slab = [&](int slab, lds_char_t *st) {
        if (slab == nk - 1 && krem < BK) {
            ga.issue_tail(st, wave, lane, krem);
            gb.issue_tail(st + OpA::BYTES, wave, lane, krem);
        } else {
            ga.issue(st, wave);
            gb.issue(st + OpA::BYTES, wave);
        }
    };
    // 16-bit tiles of at least 128 x 128 with 4 or more stages: each step
    // refills the stage consumed two steps earlier (LAG2, see the loop; on
    // the 128 x 128 kernel 1-7.5% faster, most for tn, whose transposed reads
    // of both operands made the barrier's wait for them longest; on the
    // narrow tiles 2-10% slower).  Otherwise each step refills the stage
    // consumed one step earlier.  The prologue issues the slabs the first
    // step does not issue itself.
    constexpr bool LAG2 = HALF && STAGES >= 4 && BM >= 128 && BN >= 128;
    // 16-bit 256 x 256 tiles (eight 128 x 64 waves) and 256 x 128 tiles
    // (eight 64 x 64 waves): fragments double-buffered per 16-wide k step
    // instead of per slab (the slab-wide sets do not fit beside 128
    // accumulators, and beside 64 they filled the 256 registers of a lane and
    // spilled), two stages; the prologue issues slab 0 only.  The 256 x 128
    // tile measured 3.4-10.2% faster this way than with three stages and
    // slab-wide sets for nn (2048-8192 x 1024-4096), -6.0% to +4.3% for nt,
    // bit-identical.
    constexpr bool FINE = HALF && BM == 256 && (BN == 256 || BN == 128);
    static_assert(!FINE || (STAGES == 2 && KSPLIT == 1), "the 256-row 16-bit loop uses two stages");
    // The fp32 K-group loop below, which reads each slab's fragments one
    // step ahead: for four stages (K >= 4096) and every transpose pair but
    // tn.  Against the per-slab reads, one machine, bit-identical:
    // 512^2x8192 nn/nt/tt 41.5/38.0/42.1 us against 54.1/41.9/53.0, 128^2x8192
    // 41.1 against 53.4; tn 55.1 against 51.1 (both operands m/n-contiguous,
    // eight 4-byte reads per fragment set); with three stages at K = 512
    // (512^3, 256^3) 1-8% slower.
    constexpr bool GROUPS32 = !HALF && KSPLIT > 1 && STAGES >= 4 && !(TA && !TB);
    constexpr int PRO = FINE ? 1 : (((HALF && !LAG2) || GROUPS32) ? STAGES : STAGES - 1);
#pragma unroll
    for (int s = 0; s < PRO; ++s) {
        if (s < nk) issue_slab(s, smem + s * STAGE_BYTES);
    }

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.f;

    constexpr int LOADS = OpA::LOADS + OpB::LOADS;
    if constexpr (FINE) {
        // Slab kt: k steps 0..KPW-2 run from registers, each reading the next
        // k step's fragments one before each MFMA (order pinned by
        // sched_barrier).  Then this wave waits for its loads of slab kt+1
        // and its fragment reads, and the workgroup meets at a barrier: slab
        // kt+1 is visible, and every wave is done with slab kt's stage.  The
        // last k step then runs while slab kt+1's first fragments are read
        // and slab kt+2's A is loaded into slab kt's stage; its B follows
        // during k step 0 of slab kt+1 (a load every second MFMA in both:
        // 1.6-2% faster at 4096^3, 5-7% at 3072^3 than all of them in the
        // last k step).  So no fragment read waits at a barrier, and each
        // load has at least KPW-2 k steps to land.  The reads after the last
        // slab fetch a stale stage that is never used (no branch between
        // them and the MFMAs).
        V8 fa[2][TM], fb[2][TN];
        constexpr int NL = TM * TN;              // MFMAs of one k step
        static_assert(KPW % 2 == 0, "k steps alternate between the two fragment sets");
        wait_vmcnt<0>();
        __syncthreads();                         // slab 0 visible
#pragma unroll
        for (int i = 0; i < TM; ++i) fa[0][i] = ga.frag(smem, wm0 + 32 * i, kk0, lane);
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[0][j] = gb.frag(smem + OpA::BYTES, wn0 + 32 * j, kk0, lane);
        if (nk > 1) issue_slab(1, smem + STAGE_BYTES);
        bool pend = false;                      // B's loads of a slab deferred to k step 0
        lds_char_t *pdst = smem;
        // FAST (a std::integral_constant): B's loads of this slab were
        // deferred by the previous step and the slab this step refills is a
        // whole slab before the last, so neither needs a test
        auto fine_step = [&](auto fast_tag, int kt) {
            constexpr bool FAST = decltype(fast_tag)::value;
            const lds_char_t *sA = smem + (kt % STAGES) * STAGE_BYTES;
            const lds_char_t *sB = sA + OpA::BYTES;
#pragma unroll
            for (int s = 0; s + 1 < KPW; ++s) {
                const int cur = s & 1, nxt = cur ^ 1;
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        const int f = i * TN + j;        // fragment of the next k step
                        if (s == 0) {
#pragma unroll
                            for (int l = 0; l < OpB::LOADS; ++l)
                                if (l * NL / OpB::LOADS == f && (FAST || pend)) gb.issue_one(pdst + OpA::BYTES, wave, l);
                        }
                        if (f < TM) fa[nxt][f] = ga.frag(sA, wm0 + 32 * f, kk0 + s + 1, lane);
                        else if (f < TM + TN) fb[nxt][f - TM] = gb.frag(sB, wn0 + 32 * (f - TM), kk0 + s + 1, lane);
                        acc[i][j] = mfma_32x32x16(fa[cur][i], fb[cur][j], acc[i][j]);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                if (s == 0 && (FAST || pend)) gb.advance();
            }
            wait_vmcnt<0>();
            __syncthreads();
            const int n2 = kt + 2;
            lds_char_t *dst = smem + (kt % STAGES) * STAGE_BYTES;   // slab n2's stage (two stages)
            const lds_char_t *rA = smem + ((kt + 1) % STAGES) * STAGE_BYTES;
            const lds_char_t *rB = rA + OpA::BYTES;
            const bool spread = FAST ? true : (n2 < nk && !(n2 == nk - 1 && krem < BK));
            if constexpr (!FAST) {
                if (n2 < nk && !spread) issue_slab(n2, dst);
            }
            constexpr int cur = (KPW - 1) & 1, nxt = cur ^ 1;
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int m = i * TN + j;
#pragma unroll
                    for (int l = 0; l < OpA::LOADS; ++l)
                        if (l * NL / OpA::LOADS == m && spread) ga.issue_one(dst, wave, l);
                    if (m < TM) fa[nxt][m] = ga.frag(rA, wm0 + 32 * m, kk0, lane);
                    else if (m < TM + TN) fb[nxt][m - TM] = gb.frag(rB, wn0 + 32 * (m - TM), kk0, lane);
                    acc[i][j] = mfma_32x32x16(fa[cur][i], fb[cur][j], acc[i][j]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            if (spread) ga.advance();
            pend = spread;
            pdst = dst;
        };
        // Step 0 (nothing deferred yet), then the steady state in a loop of
        // its own (steps 1 .. whole slabs - 3), then the last steps: as in
        // the loops below, bit-identical, and measured against the general
        // step alone on one machine 1-3.4% faster at 3072^3 to 8192^3 (fp16
        // and bf16) and 17% at 4096^2x512 nn.
        int kt = 0;
        if (nk > 0) fine_step(std::false_type(), kt++);
        const int nfast = (krem == BK ? nk : nk - 1) - 2;
        for (; kt < nfast; ++kt) fine_step(std::true_type(), kt);
        for (; kt < nk; ++kt) fine_step(std::false_type(), kt);
    } else if constexpr (HALF) {
        // Two fragment sets, the loop unrolled by two so that each set stays
        // in fixed registers.  The next slab's LDS reads are unconditional:
        // after the last slab they read a stale stage that is never used, so
        // that no branch separates them from the MFMAs (the compiler's LDS
        // wait bookkeeping would otherwise wait for them before the MFMAs).
        V8 fa0[KPW][TM], fb0[KPW][TN], fa1[KPW][TM], fb1[KPW][TN];
        auto read = [&](int slab, V8(&fa)[KPW][TM], V8(&fb)[KPW][TN]) {
            const lds_char_t *sA = smem + (slab % STAGES) * STAGE_BYTES;
            const lds_char_t *sB = sA + OpA::BYTES;
#pragma unroll
            for (int s = 0; s < KPW; ++s) {
#pragma unroll
                for (int i = 0; i < TM; ++i) fa[s][i] = ga.frag(sA, wm0 + 32 * i, kk0 + s, lane);
#pragma unroll
                for (int j = 0; j < TN; ++j) fb[s][j] = gb.frag(sB, wn0 + 32 * j, kk0 + s, lane);
            }
        };
        // FAST (a std::integral_constant): the step refills a whole slab that
        // is not the last, so the wait count, the choice between spread and
        // burst loads and the partial-slab test are all known at compile time
        auto step = [&](auto fast_tag, int kt, V8(&ca)[KPW][TM], V8(&cb)[KPW][TN],
                        V8(&na)[KPW][TM], V8(&nb)[KPW][TN]) {
            constexpr bool FAST = decltype(fast_tag)::value;
            // slabs issued so far: [0, min(nk, kt + PRO)); slab kt+1 must be
            // complete, in every wave's part
            constexpr int AHEAD = PRO - 2;           // slabs that may stay in flight
            if constexpr (FAST) wait_vmcnt<AHEAD * LOADS>();
            else if (kt + PRO <= nk) wait_vmcnt<AHEAD * LOADS>();
            else wait_vmcnt<0>();
            if constexpr (LAG2) {
                // A bare barrier: it does not wait for this wave's fragment
                // reads of slab kt+1 (issued in the previous step, first used
                // by the next step's MFMAs), so they complete while the waves
                // meet.  Safe because the loads issued below go into the stage
                // of slab kt-1, whose fragments every wave has consumed in its
                // MFMAs of the previous step.  The empty asm statements keep
                // the compiler from moving LDS reads across the barrier.
                asm volatile("" ::: "memory");
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
            } else {
                // the loads below go into the stage of slab kt, whose fragment
                // reads must be complete in every wave
                __syncthreads();
            }
            // slab kt+PRO goes into the stage of slab kt-1 (LAG2) or kt.  For
            // nn and nt on tiles of at least 128 x 128, a regular slab's loads
            // are spread between this slab's MFMAs, load l before MFMA
            // l*NM/LOADS: direct loads issued in a burst stall the matrix core
            // of their SIMD more than the same loads interleaved with its
            // MFMAs (measured 1-8%).  tn (both operands through transposed
            // reads) measured 3.5-6% slower spread, and the narrow tiles
            // 9-16% slower for nt (no difference for nn), so there the loads
            // go in one burst.  A partial last slab goes through registers,
            // all at once.
            constexpr bool SPREAD = !TA && BM >= 128 && BN >= 128;
            const int ns = kt + PRO;
            lds_char_t *dst = smem + (ns % STAGES) * STAGE_BYTES;
            const bool spread = FAST ? SPREAD : (SPREAD && ns < nk && !(ns == nk - 1 && krem < BK));
            if constexpr (FAST) {
                if constexpr (!SPREAD) {
                    ga.issue(dst, wave);
                    gb.issue(dst + OpA::BYTES, wave);
                }
            } else {
                if (ns < nk && !spread) issue_slab(ns, dst);
            }
            // The next slab's fragments are read between this slab's MFMAs,
            // one before each (order pinned by sched_barrier), rather than as
            // one block before them: each read then overlaps an MFMA.  Measured
            // on the 128 x 128 tile with two K groups, which has one fragment
            // per MFMA: 2-13% faster; the narrow tiles showed no difference
            // and keep the block.
            constexpr int NF = KPW * (TM + TN);
            constexpr bool SPLITRD = NF == KPW * TM * TN;
            if constexpr (!SPLITRD) read(kt + 1, na, nb);
            const lds_char_t *rA = smem + ((kt + 1) % STAGES) * STAGE_BYTES;
            const lds_char_t *rB = rA + OpA::BYTES;
            auto read_one = [&](int f) {
                const int s = f / (TM + TN), r = f % (TM + TN);
                if (r < TM) na[s][r] = ga.frag(rA, wm0 + 32 * r, kk0 + s, lane);
                else nb[s][r - TM] = gb.frag(rB, wn0 + 32 * (r - TM), kk0 + s, lane);
            };
            constexpr int NM = KPW * TM * TN;
#pragma unroll
            for (int s = 0; s < KPW; ++s)
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        const int m = (s * TM + i) * TN + j;
#pragma unroll
                        for (int l = 0; l < (SPREAD ? LOADS : 0); ++l) {
                            if (l * NM / LOADS == m && spread) {
                                if (l < OpA::LOADS) ga.issue_one(dst, wave, l);
                                else gb.issue_one(dst + OpA::BYTES, wave, l - OpA::LOADS);
                            }
                        }
                        if constexpr (SPLITRD) read_one(m);
                        acc[i][j] = mfma_32x32x16(ca[s][i], cb[s][j], acc[i][j]);
                        if constexpr (SPLITRD) __builtin_amdgcn_sched_barrier(0);
                    }
            if (spread) {
                ga.advance();
                gb.advance();
            }
        };
        if (nk > 0) {
            // slab 0 complete; slabs 1 .. PRO-1 may still be in flight
            if (nk >= PRO) wait_vmcnt<(PRO - 1) * LOADS>();
            else wait_vmcnt<0>();
            __syncthreads();
            read(0, fa0, fb0);
        }
        // The steady state first, in a loop of its own: while the slab a step
        // refills is a whole slab before the last, the step needs no bounds
        // tests, and the loop body is the MFMAs, the fragment reads, the
        // direct loads and one barrier per slab.  The last steps (the refills
        // running out, a partial last slab) go through the general step.
        // Results are bit-identical (the same operations in the same order).
        // Measured against the general step alone, one machine: fp16 and bf16
        // 2048^3 1.5-5.3% faster, 512x5632x2048 4.5-6.2%, 2048^2x8192
        // 5-12%, the 64x64 tile at 1024^2x4096 tn and nt 8-13%.
        int kt = 0;
        const int nfast = (krem == BK ? nk : nk - 1) - PRO;
        for (; kt + 1 < nfast; kt += 2) {
            step(std::true_type(), kt, fa0, fb0, fa1, fb1);
            step(std::true_type(), kt + 1, fa1, fb1, fa0, fb0);
        }
        for (; kt < nk; kt += 2) {
            step(std::false_type(), kt, fa0, fb0, fa1, fb1);
            if (kt + 1 < nk) step(std::false_type(), kt + 1, fa1, fb1, fa0, fb0);
        }
    } else if constexpr (GROUPS32) {
        // fp32 K groups: one wave per SIMD for each tile, so the fragment
        // reads of a slab would sit between the barrier and the wave's first
        // MFMA.  Instead step kt runs slab kt's MFMAs from registers and reads
        // slab kt+1's fragments between them.  At its start the wave waits
        // for slab kt+1 and meets the others at a barrier: slab kt+1 is then
        // visible, and every wave holds slab kt's fragments, so slab kt's
        // stage takes slab kt+STAGES (the prologue filled every stage).  The
        // reads after the last slab fetch a stale stage that is never used.
        constexpr int C2W = (BK / 8) / KSPLIT;    // fragment groups of this wave per slab
        constexpr int NM = C2W * 4 * TM * TN;
        f32x4 fa0[C2W][TM], fb0[C2W][TN], fa1[C2W][TM], fb1[C2W][TN];
        auto readf = [&](int slab, f32x4(&fa)[C2W][TM], f32x4(&fb)[C2W][TN]) {
            const lds_char_t *sA = smem + (slab % STAGES) * STAGE_BYTES;
            const lds_char_t *sB = sA + OpA::BYTES;
#pragma unroll
            for (int cc = 0; cc < C2W; ++cc) {
#pragma unroll
                for (int i = 0; i < TM; ++i) fa[cc][i] = ga.frag4(sA, wm0 + 32 * i, kgroup * C2W + cc, lane);
#pragma unroll
                for (int j = 0; j < TN; ++j) fb[cc][j] = gb.frag4(sB, wn0 + 32 * j, kgroup * C2W + cc, lane);
            }
        };
        auto gstep = [&](auto fast_tag, int kt, f32x4(&ca)[C2W][TM], f32x4(&cb)[C2W][TN], f32x4(&na)[C2W][TM],
                         f32x4(&nb)[C2W][TN]) {
            constexpr bool FAST = decltype(fast_tag)::value;
            // slabs issued so far: [0, min(nk, kt + STAGES)); slab kt+1 must be complete
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (FAST) wait_vmcnt<(STAGES - 2) * LOADS>();
            else if (kt + STAGES - 1 < nk) wait_vmcnt<(STAGES - 2) * LOADS>();
            else wait_vmcnt<0>();
            __syncthreads();
            const int ns = kt + STAGES;
            lds_char_t *dst = smem + (kt % STAGES) * STAGE_BYTES;      // slab kt's stage
            const bool spread = FAST ? true : (ns < nk && !(ns == nk - 1 && krem < BK));
            if constexpr (!FAST) {
                if (ns < nk && !spread) issue_slab(ns, dst);
            }
            readf(kt + 1, na, nb);
            // the reads go out before this slab's MFMAs (the compiler would
            // otherwise sink them below the MFMAs and wait for them there)
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int cc = 0; cc < C2W; ++cc)
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int j = 0; j < TN; ++j) {
                            const int m = ((cc * 4 + e) * TM + i) * TN + j;
#pragma unroll
                            for (int l = 0; l < LOADS; ++l) {
                                if (l * NM / LOADS == m && spread) {
                                    if (l < OpA::LOADS) ga.issue_one(dst, wave, l);
                                    else gb.issue_one(dst + OpA::BYTES, wave, l - OpA::LOADS);
                                }
                            }
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(ca[cc][i][e], cb[cc][j][e], acc[i][j], 0, 0,
                                                                             0);
                        }
            if (spread) {
                ga.advance();
                gb.advance();
            }
        };
        if (nk > 0) {
            // slab 0 complete; slabs 1 .. STAGES-1 may still be in flight
            if (nk >= STAGES) wait_vmcnt<(STAGES - 1) * LOADS>();
            else wait_vmcnt<0>();
            __syncthreads();
            readf(0, fa0, fb0);
        }
        // the steady state (the refilled slab a whole slab before the last)
        // in a loop of its own, then the last steps
        int kt = 0;
        const int nfast = (krem == BK ? nk : nk - 1) - STAGES;
        for (; kt + 1 < nfast; kt += 2) {
            gstep(std::true_type(), kt, fa0, fb0, fa1, fb1);
            gstep(std::true_type(), kt + 1, fa1, fb1, fa0, fb0);
        }
        for (; kt < nk; kt += 2) {
            gstep(std::false_type(), kt, fa0, fb0, fa1, fb1);
            if (kt + 1 < nk) gstep(std::false_type(), kt + 1, fa1, fb1, fa0, fb0);
        }
    } else {
        // One barrier per slab, at its start: slab kt is then in LDS for
        // every wave and every wave is done with slab kt-1, whose stage
        // receives the loads of slab kt+STAGES-1.  The slab's MFMAs follow,
        // the compiler interleaving the fragment reads with them; a wave
        // waiting at the next barrier still has its last MFMAs in flight.
        int stage = 0;
        // FAST: as in the 16-bit loop, the step refills a whole slab that is
        // not the last
        auto fstep = [&](auto fast_tag, int kt) {
            constexpr bool FAST = decltype(fast_tag)::value;
            if constexpr (FAST) wait_vmcnt<(STAGES - 2) * LOADS>();
            else if (kt + STAGES - 2 < nk) wait_vmcnt<(STAGES - 2) * LOADS>();
            else wait_vmcnt<0>();
            __syncthreads();
            // slab kt+STAGES-1 goes into the stage of slab kt-1.  A regular
            // slab's loads are spread between this slab's MFMAs (load l
            // before MFMA l*NM/LOADS): a direct load stalls its SIMD's matrix
            // core less there than in a burst after the barrier.  A partial
            // last slab goes through registers, all at once.
            const int ns = kt + STAGES - 1;
            lds_char_t *dst = smem + ((stage == 0 ? STAGES : stage) - 1) * STAGE_BYTES;   // stage of slab kt-1
            const bool spread = FAST ? true : (ns < nk && !(ns == nk - 1 && krem < BK));
            if constexpr (!FAST) {
                if (ns < nk && !spread) issue_slab(ns, dst);
            }
            const lds_char_t *sA = smem + stage * STAGE_BYTES;
            const lds_char_t *sB = sA + OpA::BYTES;
            constexpr int C2W = (BK / 8) / KSPLIT;   // fragment groups of this wave per slab
            constexpr int NM = C2W * 4 * TM * TN;
            // BK/2 MFMA steps of k = 2 per slab, fragments 4 steps at a time;
            // K group g takes fragment groups [g, g+1) * C2W
#pragma unroll
            for (int cc = 0; cc < C2W; ++cc) {
                const int c2 = (KSPLIT == 1 ? 0 : kgroup * C2W) + cc;
                f32x4 a[TM], b[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i) a[i] = ga.frag4(sA, wm0 + 32 * i, c2, lane);
#pragma unroll
                for (int j = 0; j < TN; ++j) b[j] = gb.frag4(sB, wn0 + 32 * j, c2, lane);
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int j = 0; j < TN; ++j) {
                            const int m = ((cc * 4 + e) * TM + i) * TN + j;
#pragma unroll
                            for (int l = 0; l < LOADS; ++l) {
                                if (l * NM / LOADS == m && spread) {
                                    if (l < OpA::LOADS) ga.issue_one(dst, wave, l);
                                    else gb.issue_one(dst + OpA::BYTES, wave, l - OpA::LOADS);
                                }
                            }
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][e], b[j][e], acc[i][j], 0, 0, 0);
                        }
            }
            if (spread) {
                ga.advance();
                gb.advance();
            }
            stage = (stage + 1 == STAGES) ? 0 : stage + 1;
        };
        // The steady state in a loop of its own, as in the 16-bit loop; bit-
        // identical.  Measured against the general step alone, one machine:
        // 4096^3 1.0-4.0% faster (the 4-byte-load kernel 9.7-10.4%),
        // 8192x256x8192 7.6-12.5%, 512^3 8-13%, the 128x64 tile 3%, the
        // 128x128 tile 2.5-5.6% except nt, which was 0-24% slower
        // (6144^2x2048, 3072x4096^2, 5120x4096x2048) and keeps the general
        // loop.  The 64x64 tile takes it on grids whose workgroups are all
        // resident at once: at most 1024 (four per CU) for 16-deep slabs,
        // above which it measured 3-22% slower at 2304x2048^2, 3000^3 and
        // 3072^3 (4.5 to 9 workgroups per CU); at most 768 (three per CU,
        // 48 KB of LDS each) for 32-deep slabs.
        int kt = 0;
        if constexpr (!(BM == 128 && BN == 128 && !TA && TB)) {
            const bool fast = !(BM == 64 && BN == 64) || gridDim.x * gridDim.y <= (FBK == 32 ? 768 : 1024);
            const int nfast = fast ? (krem == BK ? nk : nk - 1) - (STAGES - 1) : 0;
            for (; kt < nfast; ++kt) fstep(std::true_type(), kt);
        }
        for (; kt < nk; ++kt) fstep(std::false_type(), kt);
    }

    // ---- sum the K groups' partial accumulators (KSPLIT == 2) ---------------
    // Block q (= i*TN + j) belongs to group 0 when q < NB/2, else to group 1.
    // Each wave writes the blocks it does not own to its exchange slot, in
    // increasing q, 16 bytes per lane per 4 registers.
    __syncthreads();  // every wave is done with the ring
    if constexpr (!HALF && KSPLIT > 1) {
        fp32_groups_epilogue<KSPLIT, NWG, WAVES_N, WM, WN, EPI_LD>(p, smem, acc[0][0], wave, lane, m0, n0, split);
        return;
    }
    if constexpr (KSPLIT == 2) {
        lds_char_t *mine = smem + wave * (NB / 2) * 4096;
        const lds_char_t *theirs = smem + ((wave + NWG) % NW) * (NB / 2) * 4096;
        int w = 0;
#pragma unroll
        for (int q = 0; q < NB; ++q) {
            const bool own = (q < NB / 2) == (kgroup == 0);
            if (!own) {
#pragma unroll
                for (int c4 = 0; c4 < 4; ++c4) {
                    const f32x16 &v = acc[q / TN][q % TN];
                    const f32x4 x = {v[4 * c4], v[4 * c4 + 1], v[4 * c4 + 2], v[4 * c4 + 3]};
                    *(__attribute__((address_space(3))) f32x4 *)(mine + w * 4096 + c4 * 1024 + lane * 16) = x;
                }
                ++w;
            }
        }
        __syncthreads();
        int rd = 0;
#pragma unroll
        for (int q = 0; q < NB; ++q) {
            const bool own = (q < NB / 2) == (kgroup == 0);
            if (own) {
#pragma unroll
                for (int c4 = 0; c4 < 4; ++c4) {
                    const f32x4 x = *(const __attribute__((address_space(3))) f32x4 *)(theirs + rd * 4096 + c4 * 1024 + lane * 16);
                    f32x16 &v = acc[q / TN][q % TN];
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[4 * c4 + e] += x[e];
                }
                ++rd;
            }
        }
        __syncthreads();  // exchange slots are reused for the epilogue staging
    }

    // ---- epilogue --------------------------------------------------------------
    // Accumulator register r of lane l in a 32x32 block holds row
    // 8*(r/4) + 4*(l/32) + r%4, column l%32.  Each owned block is staged in
    // this wave's LDS slot as fp32 [32][EPI_LD]; lane l then takes row l/2,
    // columns 16*(l%2) .. +15, forms alpha*acc + beta*C + bias and the
    // activation in fp32, and writes them with 16-byte stores (one rounding to
    // the output type per element), or element by element at the matrix edge
    // or when C rows are not 16-byte aligned.  The 16-byte stores of a 16-bit
    // C carry the non-temporal hint (C is not read again by the kernel); fp32
    // C and the 256x128 tile keep plain stores, which measured faster there.
    constexpr bool HALF_C = sizeof(TC) == 2;       // 16-bit output
    constexpr bool NT_STORE = HALF_C && !(BM == 256 && BN == 128);
    // The 128 x 128 two-K-group tile with a 16-bit C stores whole 64-byte row
    // segments instead: lane l takes row 16*h + l/4 (h = 0, 1) and columns
    // 8*(l%4) .. +7, so each 16-byte store instruction writes 16 complete
    // segments (the two-stores-per-lane layout above writes every segment in
    // two halves, and the non-temporal halves reach memory as separate
    // partial writes: 11.5-13 MB written for the 8.4 MB C of 2048^3).  1-4%
    // faster at 2048^3 on every transpose pair, results bit-identical; on
    // the 256 x 256 tile 0.3-3.9% slower, on the others within noise.
    constexpr bool SEG = HALF_C && BM == 128 && BN == 128 && KSPLIT == 2;
    typedef TC VC8 __attribute__((ext_vector_type(8)));
    TC *C = (TC *)p.C;
    lds_char_t *stg = smem + wave * 32 * EPI_LD * 4;
    typedef __attribute__((address_space(3))) float lds_float_t;
    typedef __attribute__((address_space(3))) f32x4 lds_f32x4_t;
#pragma unroll
    for (int q = 0; q < NB; ++q) {
        const bool own = KSPLIT == 1 || ((q < NB / 2) == (kgroup == 0));
        if (!own) continue;
        const int i = q / TN, j = q % TN;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = 8 * (r >> 2) + (lane >> 5) * 4 + (r & 3);
            *(lds_float_t *)(stg + (row * EPI_LD + (lane & 31)) * 4) = acc[i][j][r];
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the block is staged
        __builtin_amdgcn_wave_barrier();
        if constexpr (SEG) {
            if (p.splits <= 1) {
                float v[2][8];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int lr = 16 * h + (lane >> 2), lc = (lane & 3) * 8;
#pragma unroll
                    for (int c4 = 0; c4 < 2; ++c4) {
                        const f32x4 x = *(const lds_f32x4_t *)(stg + (lr * EPI_LD + lc + 4 * c4) * 4);
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[h][4 * c4 + e] = x[e];
                    }
                }
                __builtin_amdgcn_s_waitcnt(0xc07f);  // reads done before the slot is rewritten
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int grow = m0 + wm0 + 32 * i + 16 * h + (lane >> 2);
                    const int gcol = n0 + wn0 + 32 * j + (lane & 3) * 8;
                    TC *c = C + (int64_t)grow * p.ldc + gcol;
                    if (p.c_vec && grow < p.M && gcol + 8 <= p.N) {
                        float cin[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) cin[e] = 0.f;
                        if (p.beta != 0.f) {
                            const VC8 c0 = *(const VC8 *)c;
#pragma unroll
                            for (int e = 0; e < 8; ++e) cin[e] = (float)c0[e];
                        }
                        epilogue_row<TC, 8>(p, v[h], cin, gcol);
                        VC8 o;
#pragma unroll
                        for (int e = 0; e < 8; ++e) o[e] = (TC)v[h][e];
                        __builtin_nontemporal_store(o, (VC8 *)c);
                    } else if (grow < p.M) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            if (gcol + e < p.N) {
                                const float cin = p.beta != 0.f ? (float)c[e] : 0.f;
                                c[e] = (TC)epilogue_value<TC>(p, v[h][e], cin, gcol + e);
                            }
                        }
                    }
                }
                continue;
            }
        }
        const int lr = lane >> 1, lc = (lane & 1) * 16;
        float v[16];
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
            const f32x4 x = *(const lds_f32x4_t *)(stg + (lr * EPI_LD + lc + 4 * c4) * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[4 * c4 + e] = x[e];
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // reads done before the slot is rewritten
        __builtin_amdgcn_wave_barrier();
        const int grow = m0 + wm0 + 32 * i + lr;
        const int gcol = n0 + wn0 + 32 * j + lc;
        if (p.splits > 1) {
            // raw fp32 partial sums of this split
            float *w = p.ws + ((int64_t)split * p.M + grow) * p.N + gcol;
            if (grow < p.M && gcol + 16 <= p.N && (p.N & 3) == 0) {
#pragma unroll
                for (int c4 = 0; c4 < 4; ++c4)
                    *(f32x4 *)(w + 4 * c4) = (f32x4){v[4 * c4], v[4 * c4 + 1], v[4 * c4 + 2], v[4 * c4 + 3]};
            } else if (grow < p.M) {
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    if (gcol + e < p.N) w[e] = v[e];
            }
            continue;
        }
        // alpha, beta, bias and the activation in fp32, one rounding to T
        TC *c = C + (int64_t)grow * p.ldc + gcol;
        if (p.c_vec && grow < p.M && gcol + 16 <= p.N) {
            float cin[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) cin[e] = 0.f;
            if (p.beta != 0.f) {
                if constexpr (HALF_C) {
                    const VC8 c0 = *(const VC8 *)c, c1 = *(const VC8 *)(c + 8);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        cin[e] = (float)c0[e];
                        cin[8 + e] = (float)c1[e];
                    }
                } else {
#pragma unroll
                    for (int c4 = 0; c4 < 4; ++c4) {
                        const f32x4 ci = *(const f32x4 *)(c + 4 * c4);
#pragma unroll
                        for (int e = 0; e < 4; ++e) cin[4 * c4 + e] = ci[e];
                    }
                }
            }
            epilogue_row16<TC>(p, v, cin, gcol);
            if constexpr (HALF_C) {
                VC8 o0, o1;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    o0[e] = (TC)v[e];
                    o1[e] = (TC)v[8 + e];
                }
                if constexpr (NT_STORE) {
                    __builtin_nontemporal_store(o0, (VC8 *)c);
                    __builtin_nontemporal_store(o1, (VC8 *)(c + 8));
                } else {
                    *(VC8 *)c = o0;
                    *(VC8 *)(c + 8) = o1;
                }
            } else {
#pragma unroll
                for (int c4 = 0; c4 < 4; ++c4)
                    *(f32x4 *)(c + 4 * c4) = (f32x4){v[4 * c4], v[4 * c4 + 1], v[4 * c4 + 2], v[4 * c4 + 3]};
            }
        } else if (grow < p.M) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                if (gcol + e < p.N) {
                    const float cin = p.beta != 0.f ? (float)c[e] : 0.f;
                    c[e] = (TC)epilogue_value<TC>(p, v[e], cin, gcol + e);
                }
            }
        }
    }
}

template <typename T, int BM, int BN, int WM, int WN, bool TA, bool TB, int STAGES, int KSPLIT,
          int LB = 16, typename TC = T, int FBK = 16, int LBMN = LB>
hipError_t launch_pipe(const GemmParams &p, hipStream_t s)
{
    const unsigned nwg = (unsigned)p.tiles_m * (unsigned)p.tiles_n * (unsigned)(p.splits > 1 ? p.splits : 1);
    GemmParams arg = p;
    void *args[] = {&arg};
    return hipLaunchKernel((const void *)&gemm_pipe_kernel<T, BM, BN, WM, WN, TA, TB, STAGES, KSPLIT, LB, TC, FBK, LBMN>,
                           dim3(nwg, p.batch), dim3(64 * (BM / WM) * (BN / WN) * KSPLIT), args, 0, s);
}

}  // namespace dg
