// sq_llm_int8_linear_noalloc: the LLM.int8() decomposition with its workspace
// in a fixed device array of this library instead of caller memory, for
// callers that cannot allocate (code under graph capture, tight serving
// loops). The array is a file-scope __device__ object: every GPU the library
// runs on holds its own copy for the life of the process. Host code never
// passes the array's name to a kernel (that is a host-side stand-in); its
// device address is looked up once per device with hipGetSymbolAddress, with
// that device current, and kept.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "smoothquant.h"
#include "sq_launch.h"
#include "sq_validate.h"

namespace {

static __device__ __align__(256) unsigned char scratch[SQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`.
hipError_t scratch_address(void** out) {
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev)) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) return e;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" sq_status sq_llm_int8_linear_noalloc(const void* x, sq_dtype x_dt, int64_t M, int64_t K, sq_norm norm,
                                                const float* gamma, const float* beta, float eps, float tau,
                                                const void* w, sq_dtype w_dt, const int8_t* wq,
                                                const float* w_scale, int64_t N, const float* bias, void* y,
                                                sq_dtype y_dt, void* stream) {
  sq_llm_int8_layout l{};
  if (sq_status s = sq_llm_int8_workspace(M, N, K, &l)) return s;
  // the argument checks of sq_llm_int8_linear, with a stand-in workspace that passes its own checks
  void* const stand_in = reinterpret_cast<void*>(uintptr_t{256});
  if (sq_status s = sq::check_llm_int8(x, x_dt, M, K, norm, gamma, beta, eps, tau, w, w_dt, wq, w_scale, N, bias, y,
                                       y_dt, stand_in, l.total, l.total))
    return s;
  if (l.total > SQ_NOALLOC_SCRATCH_BYTES) return SQ_ERR_TOO_LARGE;
  void* base = nullptr;
  if (scratch_address(&base) != hipSuccess) return SQ_ERR_HIP;
  char* b = static_cast<char*>(base);
  sq::LlmArgs a{x, x_dt, M, static_cast<int>(K), norm, gamma, beta, eps, tau, w, w_dt, wq, w_scale, N, bias, y, y_dt,
                reinterpret_cast<float*>(b + l.absmax), reinterpret_cast<int*>(b + l.count),
                reinterpret_cast<int*>(b + l.idx), reinterpret_cast<float*>(b + l.gamma_m),
                reinterpret_cast<float*>(b + l.beta_m), reinterpret_cast<float*>(b + l.stats),
                reinterpret_cast<int8_t*>(b + l.xq), reinterpret_cast<float*>(b + l.x_scale),
                reinterpret_cast<uint16_t*>(b + l.x16), reinterpret_cast<uint16_t*>(b + l.w16),
                reinterpret_cast<float*>(b + l.deq)};
  return sq::launch_llm_int8(a, static_cast<hipStream_t>(stream)) == hipSuccess ? SQ_OK : SQ_ERR_HIP;
}
