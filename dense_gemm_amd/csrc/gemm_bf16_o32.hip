// bf16-operand, fp32-accumulate kernels with an fp32 output (the bf16 kernels
// of gemm_tables16.hpp writing fp32 C).
#include "gemm_tables16.hpp"

namespace dg {

const launch_fn *bf16_o32_launchers(int config) { return mfma16_table<__bf16, float>(config); }
const launch_fn *bf16_o32_pipe_launchers(int config) { return pipe16_table<__bf16, float>(config); }

}  // namespace dg
