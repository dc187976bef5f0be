// The FP8 (OCP E4M3) row quantiser: the fused norm + quantise kernel with one
// step fl32(absmax / 448) per row and E4M3 codes (activations, and the fold's
// weight rows). Its own source so its instantiations compile in parallel.
#include "rows.h"

namespace sq {

hipError_t launch_norm_quant_fp8(const RowArgs& a, hipStream_t st) {
  return ModeLaunch<kRowsFp8>::run(a, nullptr, 0, st);
}

}  // namespace sq
