// Launcher tables of the 16-bit-operand kernels (fp16 or bf16 operands, fp32
// accumulation), for one operand type T and one output type TC (T itself, or
// fp32).  Each .hip file instantiates one (T, TC) pair, so the four pairs
// compile in parallel.
#pragma once

#include "gemm_mfma.hpp"
#include "gemm_pipe.hpp"

namespace dg {

// register-staged kernels (operands no pipelined kernel takes: odd row
// strides or m/n extents): [config][vec ? 0 : 4 + transA * 2 + transB]
//   0: 128x128 tile, four 64x64 waves;  1: 256x128 tile, four 128x64 waves
#define DG_MFMA8(T, TC, BM, BN, BK, WM, WN, MINW)                                               \
    {                                                                                           \
        launch_mfma<T, BM, BN, BK, WM, WN, false, false, true, MINW, TC>,                       \
        launch_mfma<T, BM, BN, BK, WM, WN, false, true, true, MINW, TC>,                        \
        launch_mfma<T, BM, BN, BK, WM, WN, true, false, true, MINW, TC>,                        \
        launch_mfma<T, BM, BN, BK, WM, WN, true, true, true, MINW, TC>,                         \
        launch_mfma<T, BM, BN, BK, WM, WN, false, false, false, MINW, TC>,                      \
        launch_mfma<T, BM, BN, BK, WM, WN, false, true, false, MINW, TC>,                       \
        launch_mfma<T, BM, BN, BK, WM, WN, true, false, false, MINW, TC>,                       \
        launch_mfma<T, BM, BN, BK, WM, WN, true, true, false, MINW, TC>,                        \
    }

template <typename T, typename TC>
const launch_fn *mfma16_table(int config)
{
    static const launch_fn table[2][8] = {
        DG_MFMA8(T, TC, 128, 128, 64, 64, 64, 1),
        DG_MFMA8(T, TC, 256, 128, 64, 128, 64, 1),
    };
    return table[config];
}
#undef DG_MFMA8

// pipelined direct-to-LDS kernels: [config][transA * 2 + transB]
//   0: 128x128 tile, 4 stages, two K groups of 4 waves (one workgroup per CU)
//   1: 256x128 tile, 3 stages, eight 64x64 waves (144 KB: one workgroup per
//      CU, as with 2 stages, whose shorter prefetch measured 8% slower)
//   2: 128x128 tile, 2 stages, two K groups (two workgroups per CU)
//   3: 64x64 tile, 4 stages, two K groups of two 64x32 waves (narrow outputs:
//      attention's N = d_head products)
//   4: 128x32 tile, 4 stages, four 32x32 waves (N = 32: low-rank products)
//   5: 32x128 tile, 4 stages, four 32x32 waves (M = 32)
//   6: 256x256 tile, 2 stages, eight 128x64 waves (large squares)
//   7, 8: configs 0 and 3 with 4-byte direct loads (rows 4-byte but not
//      16-byte aligned; the larger tiles would spill the four times as many
//      per-lane offsets)
#define DG_PIPE4(T, TC, BM, BN, WM, WN, ST, KS, LB)                                             \
    {launch_pipe<T, BM, BN, WM, WN, false, false, ST, KS, LB, TC>,                              \
     launch_pipe<T, BM, BN, WM, WN, false, true, ST, KS, LB, TC>,                               \
     launch_pipe<T, BM, BN, WM, WN, true, false, ST, KS, LB, TC>,                               \
     launch_pipe<T, BM, BN, WM, WN, true, true, ST, KS, LB, TC>}

template <typename T, typename TC>
const launch_fn *pipe16_table(int config)
{
    static const launch_fn table[9][4] = {
        DG_PIPE4(T, TC, 128, 128, 64, 64, 4, 2, 16),
        DG_PIPE4(T, TC, 256, 128, 64, 64, 2, 1, 16),
        DG_PIPE4(T, TC, 128, 128, 64, 64, 2, 2, 16),
        DG_PIPE4(T, TC, 64, 64, 64, 32, 4, 2, 16),
        DG_PIPE4(T, TC, 128, 32, 32, 32, 4, 1, 16),
        DG_PIPE4(T, TC, 32, 128, 32, 32, 4, 1, 16),
        DG_PIPE4(T, TC, 256, 256, 128, 64, 2, 1, 16),
        DG_PIPE4(T, TC, 128, 128, 64, 64, 4, 2, 4),
        DG_PIPE4(T, TC, 64, 64, 64, 32, 4, 2, 4),
    };
    return table[config];
}
#undef DG_PIPE4

}  // namespace dg
