// The FP8 per-tensor code pass: the fused norm + quantise kernel with one step
// given for the whole tensor and OCP E4M3 codes saturated to [-448, 448]
// ("SmoothQuant, in depth", "Granularity: O1, O2, O3 and what kernels run
// today", with the FP8 codes of "LLM.int8() and SmoothQuant", "example: what
// you get"). Its own source so that its instantiations compile in parallel.
#include "rows.h"

namespace sq {

hipError_t launch_rows_given_step_fp8(const RowArgs& a, const float* step, bool write_scale, hipStream_t st) {
  return ModeLaunch<kRowsFp8GivenStep>::run(a, step, write_scale ? 1 : 0, st);
}

hipError_t launch_norm_quant_fp8_given_step(const RowArgs& a, const float* step, hipStream_t st) {
  return launch_rows_given_step_fp8(a, step, true, st);
}

}  // namespace sq
