// The per-tensor code pass: the fused norm + quantise kernel with one step
// given for the whole tensor, codes clipped to [-127, 127]. Its own source so
// that its instantiations compile in parallel with the other row kernels.
#include "rows.h"

namespace sq {

hipError_t launch_rows_given_step(const RowArgs& a, const float* step, bool write_scale, hipStream_t st) {
  return ModeLaunch<kRowsGivenStep>::run(a, step, write_scale ? 1 : 0, st);
}

hipError_t launch_norm_quant_given_step(const RowArgs& a, const float* step, hipStream_t st) {
  return launch_rows_given_step(a, step, true, st);
}

}  // namespace sq
