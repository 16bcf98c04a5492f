// fp32 matrix-core kernel instantiations (v_mfma_f32_32x32x2_f32).
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

// [config][vec ? 0 : 4 + transA * 2 + transB]
const launch_fn *f32_launchers(int config)
{
    static const launch_fn table[2][8] = {
        DG_VARIANTS(float, 256, 128, 16, 128, 64, 2),
        DG_VARIANTS(float, 128, 128, 16, 64, 64, 2),
    };
    return table[config];
}

// pipelined direct-to-LDS kernels: [config][transA * 2 + transB]
//   0: 256x128 tile, 3 stages, 4 waves of 128x64 (two workgroups per CU)
//   1: 256x256 tile, 4 stages, 8 waves of 128x64 (one workgroup per CU)
//   2: 128x128 tile, 4 stages, 4 waves of 64x64 (two workgroups per CU)
//   3, 4: configs 0 and 2 with 4-byte direct loads (rows not 16-byte aligned)
//   5: 128x64 tile, 4 stages, 4 waves of 64x32 (grids too small for the
//      128x128 tile to give every compute unit one: tall-skinny outputs)
//   6: 64x64 tile, 4 stages, 4 waves of 32x32 (two or more workgroups per CU)
//   7, 8: configs 5 and 6 with 4-byte direct loads
//   9: 64x64 tile, 3 stages of 32-deep slabs (128-byte k-contiguous rows),
//      4 waves of 32x32 (three workgroups per CU)
//   10: 32x32 tile, 3 stages of 32-deep slabs, four K groups of one 32x32
//      wave (one wave per SIMD for each workgroup)
//   11: config 10 with 4 stages
//   12, 13: configs 6 and 9 for rows that are 4-byte aligned only: 16-byte
//      direct loads for a k-contiguous operand, 4-byte ones for an
//      m/n-contiguous one
#define DG_PIPE4(BM, BN, WM, WN, ST)                                                                \
    {launch_pipe<float, BM, BN, WM, WN, false, false, ST, 1>, launch_pipe<float, BM, BN, WM, WN, false, true, ST, 1>, \
     launch_pipe<float, BM, BN, WM, WN, true, false, ST, 1>, launch_pipe<float, BM, BN, WM, WN, true, true, ST, 1>}
#define DG_PIPE4DW(BM, BN, WM, WN, ST)                                                              \
    {launch_pipe<float, BM, BN, WM, WN, false, false, ST, 1, 4>, launch_pipe<float, BM, BN, WM, WN, false, true, ST, 1, 4>, \
     launch_pipe<float, BM, BN, WM, WN, true, false, ST, 1, 4>, launch_pipe<float, BM, BN, WM, WN, true, true, ST, 1, 4>}
const launch_fn *f32_pipe_launchers(int config)
{
    static const launch_fn table[14][4] = {
        {launch_pipe<float, 256, 128, 128, 64, false, false, 3, 1>, launch_pipe<float, 256, 128, 128, 64, false, true, 3, 1>,
         launch_pipe<float, 256, 128, 128, 64, true, false, 3, 1>, launch_pipe<float, 256, 128, 128, 64, true, true, 3, 1>},
        {launch_pipe<float, 256, 256, 128, 64, false, false, 4, 1>, launch_pipe<float, 256, 256, 128, 64, false, true, 4, 1>,
         launch_pipe<float, 256, 256, 128, 64, true, false, 4, 1>, launch_pipe<float, 256, 256, 128, 64, true, true, 4, 1>},
        {launch_pipe<float, 128, 128, 64, 64, false, false, 4, 1>, launch_pipe<float, 128, 128, 64, 64, false, true, 4, 1>,
         launch_pipe<float, 128, 128, 64, 64, true, false, 4, 1>, launch_pipe<float, 128, 128, 64, 64, true, true, 4, 1>},
        DG_PIPE4DW(256, 128, 128, 64, 3),
        DG_PIPE4DW(128, 128, 64, 64, 4),
        DG_PIPE4(128, 64, 64, 32, 4),
        DG_PIPE4(64, 64, 32, 32, 4),
        DG_PIPE4DW(128, 64, 64, 32, 4),
        DG_PIPE4DW(64, 64, 32, 32, 4),
        {launch_pipe<float, 64, 64, 32, 32, false, false, 3, 1, 16, float, 32>,
         launch_pipe<float, 64, 64, 32, 32, false, true, 3, 1, 16, float, 32>,
         launch_pipe<float, 64, 64, 32, 32, true, false, 3, 1, 16, float, 32>,
         launch_pipe<float, 64, 64, 32, 32, true, true, 3, 1, 16, float, 32>},
        {launch_pipe<float, 32, 32, 32, 32, false, false, 3, 4, 16, float, 32>,
         launch_pipe<float, 32, 32, 32, 32, false, true, 3, 4, 16, float, 32>,
         launch_pipe<float, 32, 32, 32, 32, true, false, 3, 4, 16, float, 32>,
         launch_pipe<float, 32, 32, 32, 32, true, true, 3, 4, 16, float, 32>},
        {launch_pipe<float, 32, 32, 32, 32, false, false, 4, 4, 16, float, 32>,
         launch_pipe<float, 32, 32, 32, 32, false, true, 4, 4, 16, float, 32>,
         launch_pipe<float, 32, 32, 32, 32, true, false, 4, 4, 16, float, 32>,
         launch_pipe<float, 32, 32, 32, 32, true, true, 4, 4, 16, float, 32>},
        {launch_pipe<float, 64, 64, 32, 32, false, false, 4, 1, 16, float, 16, 4>,
         launch_pipe<float, 64, 64, 32, 32, false, true, 4, 1, 16, float, 16, 4>,
         launch_pipe<float, 64, 64, 32, 32, true, false, 4, 1, 16, float, 16, 4>,
         launch_pipe<float, 64, 64, 32, 32, true, true, 4, 1, 16, float, 16, 4>},
        {launch_pipe<float, 64, 64, 32, 32, false, false, 3, 1, 16, float, 32, 4>,
         launch_pipe<float, 64, 64, 32, 32, false, true, 3, 1, 16, float, 32, 4>,
         launch_pipe<float, 64, 64, 32, 32, true, false, 3, 1, 16, float, 32, 4>,
         launch_pipe<float, 64, 64, 32, 32, true, true, 3, 1, 16, float, 32, 4>},
    };
    return table[config];
}
#undef DG_PIPE4
#undef DG_PIPE4DW

}  // namespace dg
