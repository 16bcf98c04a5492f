// fp16-operand, fp32-accumulate kernels with an fp16 output
// (v_mfma_f32_32x32x16_f16): the register-staged and pipelined tables of
// gemm_tables16.hpp for _Float16.
#include "gemm_tables16.hpp"

namespace dg {

const launch_fn *f16_launchers(int config) { return mfma16_table<_Float16, _Float16>(config); }
const launch_fn *f16_pipe_launchers(int config) { return pipe16_table<_Float16, _Float16>(config); }

}  // namespace dg
