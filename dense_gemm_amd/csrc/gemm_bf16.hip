// bf16-operand, fp32-accumulate kernels with a bf16 output
// (v_mfma_f32_32x32x16_bf16): the fp16 kernels' configurations
// (gemm_tables16.hpp) with bf16 elements.
#include "gemm_tables16.hpp"

namespace dg {

const launch_fn *bf16_launchers(int config) { return mfma16_table<__bf16, __bf16>(config); }
const launch_fn *bf16_pipe_launchers(int config) { return pipe16_table<__bf16, __bf16>(config); }

}  // namespace dg
