// fp16-operand, fp32-accumulate kernels with an fp32 output: the fp16 kernels
// (gemm_tables16.hpp) writing the fp32 result straight to C, with no rounding
// to fp16 ("Metal GEMM Kernels for LoRA Training on Apple Silicon", section 4,
// the fp32-output variant of its kernel).
#include "gemm_tables16.hpp"

namespace dg {

const launch_fn *f16_o32_launchers(int config) { return mfma16_table<_Float16, float>(config); }
const launch_fn *f16_o32_pipe_launchers(int config) { return pipe16_table<_Float16, float>(config); }

}  // namespace dg
