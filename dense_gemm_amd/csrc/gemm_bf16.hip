// bf16-operand, fp32-accumulate kernel instantiations
// (v_mfma_f32_32x32x16_bf16): the pipelined kernels of gemm_pipe.hpp with
// bf16 elements, in the fp16 kernels' configurations.
#include "gemm_mfma.hpp"
#include "gemm_pipe.hpp"

namespace dg {

#define DG_VARIANTS(T, BM, BN, BK, WM, WN, MINW)                                         \
    {                                                                                   \
        launch_mfma<T, BM, BN, BK, WM, WN, false, false, true, MINW>,                   \
        launch_mfma<T, BM, BN, BK, WM, WN, false, true, true, MINW>,                    \
        launch_mfma<T, BM, BN, BK, WM, WN, true, false, true, MINW>,                    \
        launch_mfma<T, BM, BN, BK, WM, WN, true, true, true, MINW>,                     \
        launch_mfma<T, BM, BN, BK, WM, WN, false, false, false, MINW>,                  \
        launch_mfma<T, BM, BN, BK, WM, WN, false, true, false, MINW>,                   \
        launch_mfma<T, BM, BN, BK, WM, WN, true, false, false, MINW>,                   \
        launch_mfma<T, BM, BN, BK, WM, WN, true, true, false, MINW>,                    \
    }

// register-staged kernels (operands no pipelined kernel takes: odd row
// strides or m/n extents): [config][vec ? 0 : 4 + transA * 2 + transB]
const launch_fn *bf16_launchers(int config)
{
    static const launch_fn table[2][8] = {
        DG_VARIANTS(__bf16, 128, 128, 64, 64, 64, 1),
        DG_VARIANTS(__bf16, 256, 128, 64, 128, 64, 1),
    };
    return table[config];
}
#undef DG_VARIANTS

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
#define DG_PIPE4(T, BM, BN, WM, WN, ST, KS)                                                   \
    {launch_pipe<T, BM, BN, WM, WN, false, false, ST, KS>, launch_pipe<T, BM, BN, WM, WN, false, true, ST, KS>, \
     launch_pipe<T, BM, BN, WM, WN, true, false, ST, KS>, launch_pipe<T, BM, BN, WM, WN, true, true, ST, KS>}
#define DG_PIPE4DW(T, BM, BN, WM, WN, ST, KS)                                                 \
    {launch_pipe<T, BM, BN, WM, WN, false, false, ST, KS, 4>, launch_pipe<T, BM, BN, WM, WN, false, true, ST, KS, 4>, \
     launch_pipe<T, BM, BN, WM, WN, true, false, ST, KS, 4>, launch_pipe<T, BM, BN, WM, WN, true, true, ST, KS, 4>}
const launch_fn *bf16_pipe_launchers(int config)
{
    static const launch_fn table[9][4] = {
        DG_PIPE4(__bf16, 128, 128, 64, 64, 4, 2),
        DG_PIPE4(__bf16, 256, 128, 64, 64, 3, 1),
        DG_PIPE4(__bf16, 128, 128, 64, 64, 2, 2),
        DG_PIPE4(__bf16, 64, 64, 64, 32, 4, 2),
        DG_PIPE4(__bf16, 128, 32, 32, 32, 4, 1),
        DG_PIPE4(__bf16, 32, 128, 32, 32, 4, 1),
        DG_PIPE4(__bf16, 256, 256, 128, 64, 2, 1),
        DG_PIPE4DW(__bf16, 128, 128, 64, 64, 4, 2),
        DG_PIPE4DW(__bf16, 64, 64, 64, 32, 4, 2),
    };
    return table[config];
}
#undef DG_PIPE4
#undef DG_PIPE4DW

}  // namespace dg
