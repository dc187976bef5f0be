// Per-tensor steps ("SmoothQuant, in depth", section "Granularity: O1, O2, O3
// and what kernels run today": per-tensor weight scales at every level, and a
// static activation scale at the fastest one; its section on failure modes:
// a static scale clips inputs outside the calibrated range).
//
//  * Per-tensor dynamic: a first row pass writes each row's max |y| into the
//    scale vector, one workgroup reduces those to the tensor's step and writes
//    it into every entry, and a second row pass writes the codes with it.
//  * Per-tensor static: one row pass with a step from calibration,
//    fl32(max_j fl32(a_j / s_j) / 127) (k_static_step), codes clipped.
//  * FP8 (OCP E4M3) takes the same passes with 448 for 127 and E4M3 codes
//    saturated to +-448.
// The scale vectors the GEMM reads then hold the one step repeated, so the
// GEMM and its epilogue are the same as for per-token / per-channel steps.
#include "rows.h"

namespace sq {

// scale[0 .. n) holds non-negative row maxima; replace every entry with the
// tensor's step fl32(max / qmax) (qmax 127 for INT8, 448 for FP8). One
// workgroup: every read precedes the barrier inside the block maximum, every
// write follows it.
__global__ __launch_bounds__(1024) void k_tensor_step(float* __restrict__ scale, int64_t n, float qmax) {
  __shared__ float red[1024 / 64];
  int m = 0;
  for (int64_t i = threadIdx.x; i < n; i += 1024) m = max(m, __float_as_int(scale[i]));
  const float step = div_rn(block_max<1024>(__int_as_float(m), red), qmax);
  for (int64_t i = threadIdx.x; i < n; i += 1024) scale[i] = step;
}

// step[0] = fl32(max_j fl32(a_j / s_j) / qmax): the smoothed input of channel j
// is y_j / s_j, so a_j / s_j is its calibration maximum (a_j >= 0, s_j > 0).
__global__ __launch_bounds__(1024) void k_static_step(const float* __restrict__ act_absmax,
                                                      const float* __restrict__ s, int K, float* __restrict__ step,
                                                      float qmax) {
  __shared__ float red[1024 / 64];
  float m = 0.0f;
  for (int j = threadIdx.x; j < K; j += 1024) m = fmaxf(m, div_rn(act_absmax[j], s[j]));
  m = block_max<1024>(m, red);
  if (threadIdx.x == 0) step[0] = div_rn(m, qmax);
}


hipError_t launch_norm_quant_per_tensor(const RowArgs& a, hipStream_t st) {
  if (hipError_t e = ModeLaunch<kRowsAmax>::run(a, nullptr, 0, st)) return e;   // x_scale[m] = max |y[m, :]|
  hipLaunchKernelGGL(k_tensor_step, dim3(1), dim3(1024), 0, st, a.x_scale, a.rows, 127.0f);
  if (hipError_t e = hipGetLastError()) return e;                               // x_scale[m] = the step
  return launch_rows_given_step(a, a.x_scale, false, st);                       // codes; x_scale as it is
}

hipError_t launch_norm_quant_fp8_per_tensor(const RowArgs& a, hipStream_t st) {
  if (hipError_t e = ModeLaunch<kRowsAmax>::run(a, nullptr, 0, st)) return e;
  hipLaunchKernelGGL(k_tensor_step, dim3(1), dim3(1024), 0, st, a.x_scale, a.rows, 448.0f);
  if (hipError_t e = hipGetLastError()) return e;
  return launch_rows_given_step_fp8(a, a.x_scale, false, st);
}

hipError_t launch_static_step(const float* act_absmax, const float* s, int K, float* step, float qmax,
                              hipStream_t st) {
  hipLaunchKernelGGL(k_static_step, dim3(1), dim3(1024), 0, st, act_absmax, s, K, step, qmax);
  return hipGetLastError();
}

}  // namespace sq
