#include "sq_validate.h"

#include <cmath>

namespace sq {
namespace {

constexpr int64_t kMaxRows = 2147483647LL;  // row indices stay in int32 inside the kernels

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool input_dtype(sq_dtype d) { return d == SQ_DT_F32 || d == SQ_DT_F16 || d == SQ_DT_BF16; }

bool norm_known(sq_norm n) { return n == SQ_NORM_NONE || n == SQ_NORM_LAYERNORM || n == SQ_NORM_RMSNORM; }

sq_status check_k(int64_t K) {
  if (K < 64 || K > SQ_K_MAX || (K % 64) != 0) return SQ_ERR_BAD_SHAPE;
  return SQ_OK;
}

sq_status check_rows(int64_t R) { return (R < 1 || R > kMaxRows) ? SQ_ERR_BAD_SHAPE : SQ_OK; }

// gamma/beta of a norm: beta only with LayerNorm; vectors 4-byte aligned.
sq_status check_norm_params(sq_norm norm, const float* gamma, const float* beta) {
  if (!norm_known(norm)) return SQ_ERR_BAD_ARG;
  if (beta && norm != SQ_NORM_LAYERNORM) return SQ_ERR_BAD_ARG;
  if (!aligned(gamma, 4) || !aligned(beta, 4)) return SQ_ERR_MISALIGNED;
  return SQ_OK;
}

}  // namespace

sq_status check_calibrate(const void* x, sq_dtype x_dt, int64_t M, int64_t K, sq_norm norm,
                          const float* gamma, const float* beta, float eps, const float* absmax) {
  if (!x || !absmax) return SQ_ERR_NULL_POINTER;
  if (!input_dtype(x_dt)) return SQ_ERR_BAD_DTYPE;
  if (sq_status s = check_rows(M)) return s;
  if (sq_status s = check_k(K)) return s;
  if (!norm_known(norm)) return SQ_ERR_BAD_ARG;
  if (norm != SQ_NORM_NONE) {
    if (sq_status s = check_norm_params(norm, gamma, beta)) return s;
    if (!(eps > 0.0f) || !std::isfinite(eps)) return SQ_ERR_BAD_ARG;
  }
  if (!aligned(x, 16) || !aligned(absmax, 4)) return SQ_ERR_MISALIGNED;
  return SQ_OK;
}

sq_status check_fold(const float* act_absmax, const void* w, sq_dtype w_dt, int64_t N, int64_t K,
                     double alpha, float eps, sq_norm norm, const float* gamma, const float* beta,
                     const float* s_out, const float* gamma_out, const float* beta_out,
                     const int8_t* wq, const float* w_scale) {
  if (!act_absmax || !w || !s_out || !gamma_out || !wq || !w_scale) return SQ_ERR_NULL_POINTER;
  if (!input_dtype(w_dt)) return SQ_ERR_BAD_DTYPE;
  if (sq_status s = check_rows(N)) return s;
  if (sq_status s = check_k(K)) return s;
  if (!(alpha >= 0.0 && alpha <= 1.0)) return SQ_ERR_BAD_ARG;
  if (!(eps > 0.0f) || !std::isfinite(eps)) return SQ_ERR_BAD_ARG;
  if (sq_status s = check_norm_params(norm, gamma, beta)) return s;
  if (norm == SQ_NORM_NONE && (gamma || beta)) return SQ_ERR_BAD_ARG;
  // beta_out exactly when there is a LayerNorm bias to fold
  if ((beta_out != nullptr) != (beta != nullptr)) return beta ? SQ_ERR_NULL_POINTER : SQ_ERR_BAD_ARG;
  if (!aligned(w, 16) || !aligned(wq, 16)) return SQ_ERR_MISALIGNED;
  if (!aligned(act_absmax, 4) || !aligned(s_out, 4) || !aligned(gamma_out, 4) || !aligned(beta_out, 4) ||
      !aligned(w_scale, 4))
    return SQ_ERR_MISALIGNED;
  return SQ_OK;
}

sq_status check_norm_quant(const void* x, sq_dtype x_dt, int64_t M, int64_t K, sq_norm norm,
                           const float* gamma_f, const float* beta_f, float eps,
                           const int8_t* xq, const float* x_scale) {
  if (!x || !xq || !x_scale) return SQ_ERR_NULL_POINTER;
  if (!input_dtype(x_dt)) return SQ_ERR_BAD_DTYPE;
  if (sq_status s = check_rows(M)) return s;
  if (sq_status s = check_k(K)) return s;
  if (sq_status s = check_norm_params(norm, gamma_f, beta_f)) return s;
  if (norm != SQ_NORM_NONE && (!(eps > 0.0f) || !std::isfinite(eps))) return SQ_ERR_BAD_ARG;
  if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(x_scale, 4)) return SQ_ERR_MISALIGNED;
  return SQ_OK;
}

sq_status check_static_step(const float* act_absmax, const float* s, int64_t K, const float* step) {
  if (!act_absmax || !s || !step) return SQ_ERR_NULL_POINTER;
  if (sq_status st = check_k(K)) return st;
  if (!aligned(act_absmax, 4) || !aligned(s, 4) || !aligned(step, 4)) return SQ_ERR_MISALIGNED;
  return SQ_OK;
}

sq_status check_gemm(const int8_t* xq, const float* x_scale, const int8_t* wq, const float* w_scale,
                     const float* bias, const void* y, sq_dtype y_dt, int64_t M, int64_t N, int64_t K) {
  if (!xq || !wq || !y) return SQ_ERR_NULL_POINTER;
  if (y_dt != SQ_DT_F32 && y_dt != SQ_DT_F16 && y_dt != SQ_DT_BF16 && y_dt != SQ_DT_I32) return SQ_ERR_BAD_DTYPE;
  if (y_dt != SQ_DT_I32 && (!x_scale || !w_scale)) return SQ_ERR_NULL_POINTER;
  if (sq_status s = check_rows(M)) return s;
  if (sq_status s = check_rows(N)) return s;
  if (sq_status s = check_k(K)) return s;
  if (!aligned(xq, 16) || !aligned(wq, 16) || !aligned(y, 16)) return SQ_ERR_MISALIGNED;
  if (!aligned(x_scale, 4) || !aligned(w_scale, 4) || !aligned(bias, 4)) return SQ_ERR_MISALIGNED;
  return SQ_OK;
}

sq_status check_llm_int8(const void* x, sq_dtype x_dt, int64_t M, int64_t K, sq_norm norm, const float* gamma,
                         const float* beta, float eps, float tau, const void* w, sq_dtype w_dt, const int8_t* wq,
                         const float* w_scale, int64_t N, const float* bias, const void* y, sq_dtype y_dt,
                         const void* workspace, uint64_t workspace_bytes, uint64_t workspace_needed) {
  if (!x || !w || !wq || !w_scale || !y || !workspace) return SQ_ERR_NULL_POINTER;
  if (!input_dtype(x_dt) || !input_dtype(w_dt)) return SQ_ERR_BAD_DTYPE;
  if (y_dt != SQ_DT_F32 && y_dt != SQ_DT_F16 && y_dt != SQ_DT_BF16) return SQ_ERR_BAD_DTYPE;
  if (sq_status s = check_rows(M)) return s;
  if (M > kLlmMaxTokens) return SQ_ERR_BAD_SHAPE;
  if (sq_status s = check_rows(N)) return s;
  if (sq_status s = check_k(K)) return s;
  if (!norm_known(norm)) return SQ_ERR_BAD_ARG;
  if (norm != SQ_NORM_NONE) {
    if (sq_status s = check_norm_params(norm, gamma, beta)) return s;
    if (!(eps > 0.0f) || !std::isfinite(eps)) return SQ_ERR_BAD_ARG;
  }
  if (!(tau >= 0.0f)) return SQ_ERR_BAD_ARG;                 // NaN or negative; +inf means no outlier
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(wq, 16) || !aligned(y, 16)) return SQ_ERR_MISALIGNED;
  if (!aligned(w_scale, 4) || !aligned(bias, 4)) return SQ_ERR_MISALIGNED;
  if (!aligned(workspace, 256)) return SQ_ERR_MISALIGNED;
  if (workspace_bytes < workspace_needed) return SQ_ERR_BAD_SHAPE;
  return SQ_OK;
}

}  // namespace sq
