// Argument checks of the C ABI. Pure C++ with no HIP calls: every check runs
// on the host before anything is launched, so the error paths work (and can be
// tested) on a machine without a GPU.
#pragma once

#include <cstdint>

#include "smoothquant.h"

namespace sq {

sq_status check_calibrate(const void* x, sq_dtype x_dt, int64_t M, int64_t K, sq_norm norm,
                          const float* gamma, const float* beta, float eps, const float* absmax);

sq_status check_fold(const float* act_absmax, const void* w, sq_dtype w_dt, int64_t N, int64_t K,
                     double alpha, float eps, sq_norm norm, const float* gamma, const float* beta,
                     const float* s_out, const float* gamma_out, const float* beta_out,
                     const int8_t* wq, const float* w_scale);

sq_status check_norm_quant(const void* x, sq_dtype x_dt, int64_t M, int64_t K, sq_norm norm,
                           const float* gamma_f, const float* beta_f, float eps,
                           const int8_t* xq, const float* x_scale);

// The static activation step from calibration maxima and smoothing factors.
sq_status check_static_step(const float* act_absmax, const float* s, int64_t K, const float* step);

sq_status check_gemm(const int8_t* xq, const float* x_scale, const int8_t* wq, const float* w_scale,
                     const float* bias, const void* y, sq_dtype y_dt, int64_t M, int64_t N, int64_t K);

// The LLM.int8() decomposition: every input as above, tau >= 0 (not NaN), the
// workspace 256-byte aligned and at least workspace_needed bytes.
constexpr int64_t kLlmMaxTokens = 64LL * 65535;            // the merge grid's token blocks
sq_status check_llm_int8(const void* x, sq_dtype x_dt, int64_t M, int64_t K, sq_norm norm, const float* gamma,
                         const float* beta, float eps, float tau, const void* w, sq_dtype w_dt, const int8_t* wq,
                         const float* w_scale, int64_t N, const float* bias, const void* y, sq_dtype y_dt,
                         const void* workspace, uint64_t workspace_bytes, uint64_t workspace_needed);

}  // namespace sq
