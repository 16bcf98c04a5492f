// bf16-operand, fp32-accumulate kernel instantiations
// (v_mfma_f32_32x32x16_bf16): the pipelined kernels of gemm_pipe.hpp with
// bf16 elements, in the fp16 kernels' configurations.
#include "gemm_pipe.hpp"

namespace dg {

// [config][transA * 2 + transB]
//   0: 128x128 tile, 4 stages, two K groups of 4 waves (one workgroup per CU)
//   1: 256x128 tile, 2 stages, eight 64x64 waves
//   2: 128x128 tile, 2 stages, two K groups (two workgroups per CU)
const launch_fn *bf16_pipe_launchers(int config)
{
    static const launch_fn table[3][4] = {
        {launch_pipe<__bf16, 128, 128, 64, 64, false, false, 4, 2>, launch_pipe<__bf16, 128, 128, 64, 64, false, true, 4, 2>,
         launch_pipe<__bf16, 128, 128, 64, 64, true, false, 4, 2>, launch_pipe<__bf16, 128, 128, 64, 64, true, true, 4, 2>},
        {launch_pipe<__bf16, 256, 128, 64, 64, false, false, 2, 1>, launch_pipe<__bf16, 256, 128, 64, 64, false, true, 2, 1>,
         launch_pipe<__bf16, 256, 128, 64, 64, true, false, 2, 1>, launch_pipe<__bf16, 256, 128, 64, 64, true, true, 2, 1>},
        {launch_pipe<__bf16, 128, 128, 64, 64, false, false, 2, 2>, launch_pipe<__bf16, 128, 128, 64, 64, false, true, 2, 2>,
         launch_pipe<__bf16, 128, 128, 64, 64, true, false, 2, 2>, launch_pipe<__bf16, 128, 128, 64, 64, true, true, 2, 2>},
    };
    return table[config];
}

}  // namespace dg
