// C ABI entry points: validate every argument, then enqueue the kernels on the
// caller's stream. Nothing here allocates, synchronises or keeps state.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "smoothquant.h"
#include "sq_launch.h"
#include "sq_validate.h"

namespace {

sq_status from_hip(hipError_t e) { return e == hipSuccess ? SQ_OK : SQ_ERR_HIP; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// Workspace regions of the LLM.int8() decomposition, each 256-byte aligned, in
// this order. The 16-bit operands are sized for every channel an outlier.
sq_llm_int8_layout llm_layout(int64_t M, int64_t N, int64_t K) {
  sq_llm_int8_layout l{};
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) {
    const uint64_t at = off;
    off = (off + bytes + 255) & ~uint64_t{255};
    return at;
  };
  const uint64_t m = static_cast<uint64_t>(M), n = static_cast<uint64_t>(N), k = static_cast<uint64_t>(K);
  l.count = take(4);
  l.idx = take(4 * k);
  l.absmax = take(4 * k);
  l.gamma_m = take(4 * k);
  l.beta_m = take(4 * k);
  l.stats = take(8 * m);
  l.xq = take(m * k);
  l.x_scale = take(4 * m);
  l.x16 = take(2 * m * k);
  l.w16 = take(2 * n * k);
  l.deq = take(4 * m * n);
  l.total = off;
  return l;
}

template <typename T>
T* at(void* base, uint64_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

}  // namespace

extern "C" {

sq_status smoothquant_calibrate(const void* x, sq_dtype x_dt, int64_t M, int64_t K, sq_norm norm,
                                const float* gamma, const float* beta, float eps, float* absmax, void* stream) {
  if (sq_status s = sq::check_calibrate(x, x_dt, M, K, norm, gamma, beta, eps, absmax)) return s;
  sq::RowArgs a{x, x_dt, M, static_cast<int>(K), norm,
                norm == SQ_NORM_NONE ? nullptr : gamma, norm == SQ_NORM_LAYERNORM ? beta : nullptr,
                eps, nullptr, nullptr, absmax};
  return from_hip(sq::launch_calibrate(a, as_stream(stream)));
}

sq_status smoothquant_fold(const float* act_absmax, const void* w, sq_dtype w_dt, int64_t N, int64_t K,
                           double alpha, float eps, sq_norm norm, const float* gamma, const float* beta,
                           float* s_out, float* gamma_out, float* beta_out, int8_t* wq, float* w_scale,
                           void* stream) {
  if (sq_status s = sq::check_fold(act_absmax, w, w_dt, N, K, alpha, eps, norm, gamma, beta, s_out, gamma_out,
                                   beta_out, wq, w_scale))
    return s;
  hipStream_t st = as_stream(stream);
  sq::FoldArgs f{act_absmax, w, w_dt, N, K, alpha, eps, gamma, beta, s_out, gamma_out, beta_out};
  if (sq_status s = from_hip(sq::launch_fold_colmax_scales(f, st))) return s;
  // W-hat = fl32(W * s) quantised per output row: the NONE-norm quantiser with gamma = s.
  sq::RowArgs q{w, w_dt, N, static_cast<int>(K), SQ_NORM_NONE, s_out, nullptr, 1.0f, wq, w_scale, nullptr};
  return from_hip(sq::launch_norm_quant(q, st));
}

sq_status sq_norm_quant(const void* x, sq_dtype x_dt, int64_t M, int64_t K, sq_norm norm, const float* gamma_f,
                        const float* beta_f, float eps, int8_t* xq, float* x_scale, void* stream) {
  if (sq_status s = sq::check_norm_quant(x, x_dt, M, K, norm, gamma_f, beta_f, eps, xq, x_scale)) return s;
  sq::RowArgs a{x, x_dt, M, static_cast<int>(K), norm, gamma_f, beta_f, eps, xq, x_scale, nullptr};
  return from_hip(sq::launch_norm_quant(a, as_stream(stream)));
}

sq_status sq_w8a8_gemm(const int8_t* xq, const float* x_scale, const int8_t* wq, const float* w_scale,
                       const float* bias, void* y, sq_dtype y_dt, int64_t M, int64_t N, int64_t K, void* stream) {
  if (sq_status s = sq::check_gemm(xq, x_scale, wq, w_scale, bias, y, y_dt, M, N, K)) return s;
  sq::GemmArgs g{xq, x_scale, wq, w_scale, y_dt == SQ_DT_I32 ? nullptr : bias, y, y_dt,
                 static_cast<int>(M), static_cast<int>(N), static_cast<int>(K)};
  return from_hip(sq::launch_gemm(g, as_stream(stream)));
}

sq_status sq_norm_quant_per_tensor(const void* x, sq_dtype x_dt, int64_t M, int64_t K, sq_norm norm,
                                   const float* gamma_f, const float* beta_f, float eps, int8_t* xq, float* x_scale,
                                   void* stream) {
  if (sq_status s = sq::check_norm_quant(x, x_dt, M, K, norm, gamma_f, beta_f, eps, xq, x_scale)) return s;
  sq::RowArgs a{x, x_dt, M, static_cast<int>(K), norm, gamma_f, beta_f, eps, xq, x_scale, nullptr};
  return from_hip(sq::launch_norm_quant_per_tensor(a, as_stream(stream)));
}

sq_status sq_norm_quant_static(const void* x, sq_dtype x_dt, int64_t M, int64_t K, sq_norm norm,
                               const float* gamma_f, const float* beta_f, float eps, const float* step, int8_t* xq,
                               float* x_scale, void* stream) {
  if (sq_status s = sq::check_norm_quant(x, x_dt, M, K, norm, gamma_f, beta_f, eps, xq, x_scale)) return s;
  if (!step) return SQ_ERR_NULL_POINTER;
  if (reinterpret_cast<uintptr_t>(step) % 4 != 0) return SQ_ERR_MISALIGNED;
  sq::RowArgs a{x, x_dt, M, static_cast<int>(K), norm, gamma_f, beta_f, eps, xq, x_scale, nullptr};
  return from_hip(sq::launch_norm_quant_given_step(a, step, as_stream(stream)));
}

sq_status sq_static_step(const float* act_absmax, const float* s, int64_t K, float* step, void* stream) {
  if (sq_status st = sq::check_static_step(act_absmax, s, K, step)) return st;
  return from_hip(sq::launch_static_step(act_absmax, s, static_cast<int>(K), step, 127.0f, as_stream(stream)));
}

sq_status smoothquant_fold_per_tensor(const float* act_absmax, const void* w, sq_dtype w_dt, int64_t N, int64_t K,
                                      double alpha, float eps, sq_norm norm, const float* gamma, const float* beta,
                                      float* s_out, float* gamma_out, float* beta_out, int8_t* wq, float* w_scale,
                                      void* stream) {
  if (sq_status s = sq::check_fold(act_absmax, w, w_dt, N, K, alpha, eps, norm, gamma, beta, s_out, gamma_out,
                                   beta_out, wq, w_scale))
    return s;
  hipStream_t st = as_stream(stream);
  sq::FoldArgs f{act_absmax, w, w_dt, N, K, alpha, eps, gamma, beta, s_out, gamma_out, beta_out};
  if (sq_status s = from_hip(sq::launch_fold_colmax_scales(f, st))) return s;
  sq::RowArgs q{w, w_dt, N, static_cast<int>(K), SQ_NORM_NONE, s_out, nullptr, 1.0f, wq, w_scale, nullptr};
  return from_hip(sq::launch_norm_quant_per_tensor(q, st));
}

sq_status sq_norm_quant_fp8(const void* x, sq_dtype x_dt, int64_t M, int64_t K, sq_norm norm, const float* gamma_f,
                            const float* beta_f, float eps, uint8_t* xq, float* x_scale, void* stream) {
  int8_t* q = reinterpret_cast<int8_t*>(xq);
  if (sq_status s = sq::check_norm_quant(x, x_dt, M, K, norm, gamma_f, beta_f, eps, q, x_scale)) return s;
  sq::RowArgs a{x, x_dt, M, static_cast<int>(K), norm, gamma_f, beta_f, eps, q, x_scale, nullptr};
  return from_hip(sq::launch_norm_quant_fp8(a, as_stream(stream)));
}

sq_status smoothquant_fold_fp8(const float* act_absmax, const void* w, sq_dtype w_dt, int64_t N, int64_t K,
                               double alpha, float eps, sq_norm norm, const float* gamma, const float* beta,
                               float* s_out, float* gamma_out, float* beta_out, uint8_t* wq, float* w_scale,
                               void* stream) {
  int8_t* q = reinterpret_cast<int8_t*>(wq);
  if (sq_status s = sq::check_fold(act_absmax, w, w_dt, N, K, alpha, eps, norm, gamma, beta, s_out, gamma_out,
                                   beta_out, q, w_scale))
    return s;
  hipStream_t st = as_stream(stream);
  sq::FoldArgs f{act_absmax, w, w_dt, N, K, alpha, eps, gamma, beta, s_out, gamma_out, beta_out};
  if (sq_status s = from_hip(sq::launch_fold_colmax_scales(f, st))) return s;
  sq::RowArgs r{w, w_dt, N, static_cast<int>(K), SQ_NORM_NONE, s_out, nullptr, 1.0f, q, w_scale, nullptr};
  return from_hip(sq::launch_norm_quant_fp8(r, st));
}

sq_status sq_fp8_gemm(const uint8_t* xq, const float* x_scale, const uint8_t* wq, const float* w_scale,
                      const float* bias, void* y, sq_dtype y_dt, int64_t M, int64_t N, int64_t K, void* stream) {
  const int8_t* xa = reinterpret_cast<const int8_t*>(xq);
  const int8_t* wa = reinterpret_cast<const int8_t*>(wq);
  if (y_dt == SQ_DT_I32) return SQ_ERR_BAD_DTYPE;
  if (sq_status s = sq::check_gemm(xa, x_scale, wa, w_scale, bias, y, y_dt, M, N, K)) return s;
  if (K % 128 != 0) return SQ_ERR_BAD_SHAPE;
  sq::GemmArgs g{xa, x_scale, wa, w_scale, bias, y, y_dt, static_cast<int>(M), static_cast<int>(N),
                 static_cast<int>(K)};
  return from_hip(sq::launch_gemm_fp8(g, as_stream(stream)));
}

sq_status sq_norm_quant_fp8_per_tensor(const void* x, sq_dtype x_dt, int64_t M, int64_t K, sq_norm norm,
                                       const float* gamma_f, const float* beta_f, float eps, uint8_t* xq,
                                       float* x_scale, void* stream) {
  int8_t* q = reinterpret_cast<int8_t*>(xq);
  if (sq_status s = sq::check_norm_quant(x, x_dt, M, K, norm, gamma_f, beta_f, eps, q, x_scale)) return s;
  sq::RowArgs a{x, x_dt, M, static_cast<int>(K), norm, gamma_f, beta_f, eps, q, x_scale, nullptr};
  return from_hip(sq::launch_norm_quant_fp8_per_tensor(a, as_stream(stream)));
}

sq_status sq_norm_quant_fp8_static(const void* x, sq_dtype x_dt, int64_t M, int64_t K, sq_norm norm,
                                   const float* gamma_f, const float* beta_f, float eps, const float* step,
                                   uint8_t* xq, float* x_scale, void* stream) {
  int8_t* q = reinterpret_cast<int8_t*>(xq);
  if (sq_status s = sq::check_norm_quant(x, x_dt, M, K, norm, gamma_f, beta_f, eps, q, x_scale)) return s;
  if (!step) return SQ_ERR_NULL_POINTER;
  if (reinterpret_cast<uintptr_t>(step) % 4 != 0) return SQ_ERR_MISALIGNED;
  sq::RowArgs a{x, x_dt, M, static_cast<int>(K), norm, gamma_f, beta_f, eps, q, x_scale, nullptr};
  return from_hip(sq::launch_norm_quant_fp8_given_step(a, step, as_stream(stream)));
}

sq_status sq_static_step_fp8(const float* act_absmax, const float* s, int64_t K, float* step, void* stream) {
  if (sq_status st = sq::check_static_step(act_absmax, s, K, step)) return st;
  return from_hip(sq::launch_static_step(act_absmax, s, static_cast<int>(K), step, 448.0f, as_stream(stream)));
}

sq_status smoothquant_fold_fp8_per_tensor(const float* act_absmax, const void* w, sq_dtype w_dt, int64_t N,
                                          int64_t K, double alpha, float eps, sq_norm norm, const float* gamma,
                                          const float* beta, float* s_out, float* gamma_out, float* beta_out,
                                          uint8_t* wq, float* w_scale, void* stream) {
  int8_t* q = reinterpret_cast<int8_t*>(wq);
  if (sq_status s = sq::check_fold(act_absmax, w, w_dt, N, K, alpha, eps, norm, gamma, beta, s_out, gamma_out,
                                   beta_out, q, w_scale))
    return s;
  hipStream_t st = as_stream(stream);
  sq::FoldArgs f{act_absmax, w, w_dt, N, K, alpha, eps, gamma, beta, s_out, gamma_out, beta_out};
  if (sq_status s = from_hip(sq::launch_fold_colmax_scales(f, st))) return s;
  sq::RowArgs r{w, w_dt, N, static_cast<int>(K), SQ_NORM_NONE, s_out, nullptr, 1.0f, q, w_scale, nullptr};
  return from_hip(sq::launch_norm_quant_fp8_per_tensor(r, st));
}

sq_status sq_llm_int8_workspace(int64_t M, int64_t N, int64_t K, sq_llm_int8_layout* layout) {
  if (!layout) return SQ_ERR_NULL_POINTER;
  if (M < 1 || M > sq::kLlmMaxTokens || N < 1 || N > 2147483647LL || K < 64 || K > SQ_K_MAX || K % 64 != 0)
    return SQ_ERR_BAD_SHAPE;
  *layout = llm_layout(M, N, K);
  return SQ_OK;
}

sq_status sq_llm_int8_linear(const void* x, sq_dtype x_dt, int64_t M, int64_t K, sq_norm norm, const float* gamma,
                             const float* beta, float eps, float tau, const void* w, sq_dtype w_dt,
                             const int8_t* wq, const float* w_scale, int64_t N, const float* bias, void* y,
                             sq_dtype y_dt, void* workspace, uint64_t workspace_bytes, void* stream) {
  const bool shape_ok = M >= 1 && M <= sq::kLlmMaxTokens && N >= 1 && K >= 64 && K <= SQ_K_MAX && K % 64 == 0;
  const uint64_t need = shape_ok ? llm_layout(M, N, K).total : 0;
  if (sq_status s = sq::check_llm_int8(x, x_dt, M, K, norm, gamma, beta, eps, tau, w, w_dt, wq, w_scale, N, bias, y,
                                       y_dt, workspace, workspace_bytes, need))
    return s;
  const sq_llm_int8_layout l = llm_layout(M, N, K);
  sq::LlmArgs a{x, x_dt, M, static_cast<int>(K), norm, gamma, beta, eps, tau, w, w_dt, wq, w_scale, N, bias, y, y_dt,
                at<float>(workspace, l.absmax), at<int>(workspace, l.count), at<int>(workspace, l.idx),
                at<float>(workspace, l.gamma_m), at<float>(workspace, l.beta_m), at<float>(workspace, l.stats),
                at<int8_t>(workspace, l.xq), at<float>(workspace, l.x_scale), at<uint16_t>(workspace, l.x16),
                at<uint16_t>(workspace, l.w16), at<float>(workspace, l.deq)};
  return from_hip(sq::launch_llm_int8(a, as_stream(stream)));
}

const char* sq_status_string(sq_status s) {
  switch (s) {
    case SQ_OK: return "SQ_OK";
    case SQ_ERR_NULL_POINTER: return "SQ_ERR_NULL_POINTER: a required pointer is NULL";
    case SQ_ERR_BAD_DTYPE: return "SQ_ERR_BAD_DTYPE: dtype not allowed for this argument";
    case SQ_ERR_BAD_SHAPE: return "SQ_ERR_BAD_SHAPE: need 1 <= M, N < 2^31 and 64 <= K <= 133120 with K % 64 == 0";
    case SQ_ERR_MISALIGNED: return "SQ_ERR_MISALIGNED: matrices need 16-byte, vectors 4-byte alignment";
    case SQ_ERR_BAD_ARG: return "SQ_ERR_BAD_ARG: alpha, eps, norm or pointer combination not allowed";
    case SQ_ERR_UNSUPPORTED: return "SQ_ERR_UNSUPPORTED: not implemented by this build";
    case SQ_ERR_HIP: return "SQ_ERR_HIP: the HIP runtime refused a launch";
    case SQ_ERR_TOO_LARGE:
      return "SQ_ERR_TOO_LARGE: the call needs more than the SQ_NOALLOC_SCRATCH_BYTES (128 MiB) of fixed scratch";
  }
  return "unknown sq_status";
}

}  // extern "C"
