// Host-side launchers of the HIP kernels (argument bundles already validated).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "smoothquant.h"

namespace sq {

// norm + quantise (xq, x_scale) or calibration (absmax) over `rows` rows of K.
struct RowArgs {
  const void* x;
  sq_dtype dtype;
  int64_t rows;
  int K;
  sq_norm norm;
  const float* gamma;
  const float* beta;
  float eps;
  int8_t* xq;
  float* x_scale;
  float* absmax;
  float* stats = nullptr;   // (mean, rstd) per row, written by the norm-statistics launch only
};

struct FoldArgs {
  const float* act_absmax;
  const void* w;
  sq_dtype dtype;
  int64_t N, K;
  double alpha;
  float eps;
  const float* gamma;
  const float* beta;
  float* s_out;
  float* gamma_out;
  float* beta_out;
};

struct GemmArgs {
  const int8_t* xq;
  const float* x_scale;
  const int8_t* wq;
  const float* w_scale;
  const float* bias;
  void* y;
  sq_dtype y_dt;
  int M, N, K;
};

// The LLM.int8() decomposition: inputs, output, and the workspace regions it uses.
struct LlmArgs {
  const void* x;
  sq_dtype x_dt;
  int64_t M;
  int K;
  sq_norm norm;
  const float* gamma;
  const float* beta;
  float eps;
  float tau;
  const void* w;
  sq_dtype w_dt;
  const int8_t* wq;
  const float* w_scale;
  int64_t N;
  const float* bias;
  void* y;
  sq_dtype y_dt;
  // workspace
  float* absmax;      // [K]
  int* count;         // [1]
  int* idx;           // [K]
  float* gamma_m;     // [K]
  float* beta_m;      // [K]
  float* stats;       // [2 M]
  int8_t* xq;         // [M, K]
  float* x_scale;     // [M]
  uint16_t* x16;      // [M, K] at most
  uint16_t* w16;      // [N, K] at most
  float* deq;         // [M, N]
};

hipError_t launch_norm_quant(const RowArgs& a, hipStream_t st);
hipError_t launch_llm_int8(const LlmArgs& l, hipStream_t st);
hipError_t launch_calibrate(const RowArgs& a, hipStream_t st);
// Column maxima of W into s_out, then s, gamma', beta' (the weight codes are a
// norm_quant pass over W with gamma = s).
hipError_t launch_fold_colmax_scales(const FoldArgs& f, hipStream_t st);
hipError_t launch_gemm(const GemmArgs& g, hipStream_t st);
// FP8 (OCP E4M3) variants: per-row steps absmax / 448 and E4M3 codes (xq, wq hold
// the code bytes); the GEMM accumulates in binary32 and needs K % 128 == 0.
hipError_t launch_norm_quant_fp8(const RowArgs& a, hipStream_t st);
hipError_t launch_gemm_fp8(const GemmArgs& g, hipStream_t st);
// One step for the whole tensor: the rows' maxima, their max, then the codes;
// x_scale ends holding the step in every entry.
hipError_t launch_norm_quant_per_tensor(const RowArgs& a, hipStream_t st);
// Codes with the step *step (device), clipped; x_scale[m] = *step.
hipError_t launch_norm_quant_given_step(const RowArgs& a, const float* step, hipStream_t st);
// As above; x_scale is written only if write_scale (it may then be the step's own buffer).
hipError_t launch_rows_given_step(const RowArgs& a, const float* step, bool write_scale, hipStream_t st);
// *step = fl32(max_j fl32(act_absmax[j] / s[j]) / qmax), qmax 127 (INT8) or 448 (FP8).
hipError_t launch_static_step(const float* act_absmax, const float* s, int K, float* step, float qmax,
                              hipStream_t st);
// FP8 with one step for the whole tensor (E4M3 codes saturated to +-448): the
// dynamic per-tensor passes with 448 for 127, and the code pass with a given step.
hipError_t launch_norm_quant_fp8_per_tensor(const RowArgs& a, hipStream_t st);
hipError_t launch_norm_quant_fp8_given_step(const RowArgs& a, const float* step, hipStream_t st);
hipError_t launch_rows_given_step_fp8(const RowArgs& a, const float* step, bool write_scale, hipStream_t st);

}  // namespace sq
