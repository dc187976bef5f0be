// Row-streaming kernels: fused norm + per-token INT8 quantisation, calibration
// absmax, and the three steps of the offline fold (weight column maxima,
// smoothing factors, per-output-channel weight quantisation).
//
// One workgroup owns one row (or a few rows for calibration); the row stays in
// registers between the statistics, the normalisation and the quantisation, so
// each element is read from HBM once and its code written once.
#include "sq_device.h"
#include "sq_launch.h"
#include "smoothquant.h"

namespace sq {

// Load one row (K elements, K % 64 == 0) into registers and apply the norm.
// On return v holds y as binary32: LayerNorm ((x - mean) * rstd) * gamma + beta,
// RMSNorm (x * rstd) * gamma, or x * gamma; a NULL gamma/beta means 1/0. The
// statistics are summed in binary64 in a fixed order and rounded once to
// binary32; rstd = fl32(1 / fl32(sqrt(fl32(var + eps)))).
template <typename T, int NORM, int NV, int THREADS>
__device__ __forceinline__ void row_y(const char* __restrict__ xrow, int K, const float* __restrict__ gamma,
                                      const float* __restrict__ beta, float eps, float (&v)[NV][8],
                                      double* red) {
  constexpr int B = Storage<T>::kBytes;
  const int nvec = K >> 3;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int vi = threadIdx.x + i * THREADS;
    if (vi < nvec) {
      load8<T>(xrow + static_cast<size_t>(vi) * 8 * B, v[i]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[i][e] = 0.0f;
    }
  }
  float mu = 0.0f, r = 1.0f;
  if constexpr (NORM == SQ_NORM_LAYERNORM) {
    double s1 = 0.0;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) s1 += static_cast<double>(v[i][e]);   // padding holds zeros
    s1 = block_sum<THREADS>(s1, red);
    const double mean = s1 / static_cast<double>(K);
    double s2 = 0.0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      if (static_cast<int>(threadIdx.x) + i * THREADS < nvec) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const double d = static_cast<double>(v[i][e]) - mean;
          s2 = __builtin_fma(d, d, s2);
        }
      }
    }
    s2 = block_sum<THREADS>(s2, red);
    mu = static_cast<float>(mean);
    const float var = static_cast<float>(s2 / static_cast<double>(K));
    r = div_rn(1.0f, sqrt_rn(add_rn(var, eps)));
  } else if constexpr (NORM == SQ_NORM_RMSNORM) {
    double s2 = 0.0;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double d = static_cast<double>(v[i][e]);
        s2 = __builtin_fma(d, d, s2);
      }
    s2 = block_sum<THREADS>(s2, red);
    const float var = static_cast<float>(s2 / static_cast<double>(K));
    r = div_rn(1.0f, sqrt_rn(add_rn(var, eps)));
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int vi = threadIdx.x + i * THREADS;
    if (vi >= nvec) continue;
    float g[8], b[8];
    if (gamma) {
      const float4 g0 = reinterpret_cast<const float4*>(gamma)[2 * vi];
      const float4 g1 = reinterpret_cast<const float4*>(gamma)[2 * vi + 1];
      g[0] = g0.x; g[1] = g0.y; g[2] = g0.z; g[3] = g0.w; g[4] = g1.x; g[5] = g1.y; g[6] = g1.z; g[7] = g1.w;
    }
    if (NORM == SQ_NORM_LAYERNORM && beta) {
      const float4 b0 = reinterpret_cast<const float4*>(beta)[2 * vi];
      const float4 b1 = reinterpret_cast<const float4*>(beta)[2 * vi + 1];
      b[0] = b0.x; b[1] = b0.y; b[2] = b0.z; b[3] = b0.w; b[4] = b1.x; b[5] = b1.y; b[6] = b1.z; b[7] = b1.w;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float t = v[i][e];
      if constexpr (NORM == SQ_NORM_LAYERNORM) t = mul_rn(sub_rn(t, mu), r);
      if constexpr (NORM == SQ_NORM_RMSNORM) t = mul_rn(t, r);
      if (gamma) t = mul_rn(t, g[e]);
      if (NORM == SQ_NORM_LAYERNORM && beta) t = add_rn(t, b[e]);
      v[i][e] = t;
    }
  }
}

// Fused norm + per-token quantisation: one workgroup per row.
template <typename T, int NORM, int NV, int THREADS>
__global__ __launch_bounds__(THREADS) void k_norm_quant(const void* __restrict__ x, int K,
                                                        const float* __restrict__ gamma,
                                                        const float* __restrict__ beta, float eps,
                                                        int8_t* __restrict__ xq, float* __restrict__ x_scale) {
  __shared__ double red[THREADS / kWave];
  const int64_t row = blockIdx.x;
  const char* xrow = static_cast<const char*>(x) + row * K * Storage<T>::kBytes;
  float v[NV][8];
  row_y<T, NORM, NV, THREADS>(xrow, K, gamma, beta, eps, v, red);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[i][e]));
  amax = block_max<THREADS>(amax, reinterpret_cast<float*>(red));
  const float step = int8_step(amax);
  if (threadIdx.x == 0) x_scale[row] = step;
  const Quantizer qz(step);
  int8_t* qrow = xq + row * K;
  const int nvec = K >> 3;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int vi = threadIdx.x + i * THREADS;
    if (vi < nvec) *reinterpret_cast<uint2*>(qrow + static_cast<size_t>(vi) * 8) = qz.codes8(v[i]);
  }
}

// Calibration: each workgroup normalises `rows` consecutive rows, keeps the
// per-column max of |y| in registers and merges it into absmax with an
// order-free atomic max.
template <typename T, int NORM, int NV, int THREADS>
__global__ __launch_bounds__(THREADS) void k_calibrate(const void* __restrict__ x, int M, int K, int rows,
                                                       const float* __restrict__ gamma,
                                                       const float* __restrict__ beta, float eps,
                                                       float* __restrict__ absmax) {
  __shared__ double red[THREADS / kWave];
  float cm[NV][8];
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) cm[i][e] = 0.0f;
  const int r0 = blockIdx.x * rows;
  const int r1 = min(M, r0 + rows);
  for (int r = r0; r < r1; ++r) {
    const char* xrow = static_cast<const char*>(x) + static_cast<int64_t>(r) * K * Storage<T>::kBytes;
    float v[NV][8];
    row_y<T, NORM, NV, THREADS>(xrow, K, gamma, beta, eps, v, red);
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) cm[i][e] = fmaxf(cm[i][e], fabsf(v[i][e]));
  }
  const int nvec = K >> 3;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int vi = threadIdx.x + i * THREADS;
    if (vi < nvec)
#pragma unroll
      for (int e = 0; e < 8; ++e) atomic_max_nonneg(absmax + vi * 8 + e, cm[i][e]);
  }
}

// Fold step 1: colmax[j] = max_n |W[n, j]| (colmax pre-zeroed). Each thread owns
// 8 adjacent columns and walks `rows` rows; the column maxima merge by atomic max.
template <typename T>
__global__ __launch_bounds__(256) void k_colmax(const void* __restrict__ w, int N, int K, int rows,
                                                float* __restrict__ colmax) {
  const int vi = blockIdx.x * 256 + threadIdx.x;
  if (vi >= (K >> 3)) return;
  const int r0 = blockIdx.y * rows;
  const int r1 = min(N, r0 + rows);
  constexpr int B = Storage<T>::kBytes;
  const char* base = static_cast<const char*>(w) + static_cast<size_t>(vi) * 8 * B;
  float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int r = r0;
  for (; r + 4 <= r1; r += 4) {
    float v[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) load8<T>(base + static_cast<int64_t>(r + u) * K * B, v[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) m[e] = fmaxf(m[e], fabsf(v[u][e]));
  }
  for (; r < r1; ++r) {
    float v[8];
    load8<T>(base + static_cast<int64_t>(r) * K * B, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) m[e] = fmaxf(m[e], fabsf(v[e]));
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) atomic_max_nonneg(colmax + vi * 8 + e, m[e]);
}

__global__ void k_fill_zero(float* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

// Fold step 2: s_j = max(fl32(max(a_j, eps)^alpha / max(w_j, eps)^(1 - alpha)), eps)
// with the quotient in binary64; gamma' = gamma / s (1 / s without gamma),
// beta' = beta / s. s_io holds the column maxima on entry and s on exit.
__global__ void k_scales(const float* __restrict__ act_absmax, float* __restrict__ s_io, int K, double alpha,
                         float eps, const float* __restrict__ gamma, const float* __restrict__ beta,
                         float* __restrict__ gamma_out, float* __restrict__ beta_out) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= K) return;
  const float a1 = fmaxf(act_absmax[j], eps);
  const float w1 = fmaxf(s_io[j], eps);
  const double q = pow(static_cast<double>(a1), alpha) / pow(static_cast<double>(w1), 1.0 - alpha);
  const float s = fmaxf(static_cast<float>(q), eps);
  s_io[j] = s;
  gamma_out[j] = div_rn(gamma ? gamma[j] : 1.0f, s);
  if (beta_out) beta_out[j] = div_rn(beta[j], s);
}

// ----------------------------------------------------------------------------- launchers

namespace {

struct RowCfg { int threads, nv; };

// Smallest (threads, vectors per thread) covering K/8 vectors, keeping at most
// ~80 binary32 values per thread in registers.
RowCfg row_cfg(int K) {
  const int nvec = K >> 3;
  static const RowCfg table[] = {{256, 1}, {256, 2}, {256, 3}, {256, 4}, {512, 3},  {512, 4},   {512, 5},
                                 {512, 6}, {1024, 4}, {1024, 6}, {1024, 8}, {1024, 10}, {1024, 13}, {1024, 17}};
  for (const RowCfg& c : table)
    if (c.threads * c.nv >= nvec) return c;
  return {1024, 17};
}

template <typename T, int NORM, int NV, int THREADS>
hipError_t launch_nq(const RowArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((k_norm_quant<T, NORM, NV, THREADS>), dim3(a.rows), dim3(THREADS), 0, st, a.x, a.K,
                     a.gamma, a.beta, a.eps, a.xq, a.x_scale);
  return hipGetLastError();
}

template <typename T, int NORM, int NV, int THREADS>
hipError_t launch_cal(const RowArgs& a, hipStream_t st) {
  const int per = 4;
  const int blocks = static_cast<int>((a.rows + per - 1) / per);
  hipLaunchKernelGGL((k_calibrate<T, NORM, NV, THREADS>), dim3(blocks), dim3(THREADS), 0, st, a.x,
                     static_cast<int>(a.rows), a.K, per, a.gamma, a.beta, a.eps, a.absmax);
  return hipGetLastError();
}

template <bool CAL, typename T, int NORM, int NV, int THREADS>
hipError_t dispatch_one(const RowArgs& a, hipStream_t st) {
  return CAL ? launch_cal<T, NORM, NV, THREADS>(a, st) : launch_nq<T, NORM, NV, THREADS>(a, st);
}

template <bool CAL, typename T, int NORM>
hipError_t dispatch_cfg(const RowArgs& a, hipStream_t st) {
  const RowCfg c = row_cfg(a.K);
#define SQ_ROW_CASE(TH, NVV) \
  if (c.threads == TH && c.nv == NVV) return dispatch_one<CAL, T, NORM, NVV, TH>(a, st);
  SQ_ROW_CASE(256, 1) SQ_ROW_CASE(256, 2) SQ_ROW_CASE(256, 3) SQ_ROW_CASE(256, 4)
  SQ_ROW_CASE(512, 3) SQ_ROW_CASE(512, 4) SQ_ROW_CASE(512, 5) SQ_ROW_CASE(512, 6)
  SQ_ROW_CASE(1024, 4) SQ_ROW_CASE(1024, 6) SQ_ROW_CASE(1024, 8) SQ_ROW_CASE(1024, 10)
  SQ_ROW_CASE(1024, 13) SQ_ROW_CASE(1024, 17)
#undef SQ_ROW_CASE
  return hipErrorInvalidValue;
}

template <bool CAL, typename T>
hipError_t dispatch_norm(const RowArgs& a, hipStream_t st) {
  switch (a.norm) {
    case SQ_NORM_NONE: return dispatch_cfg<CAL, T, SQ_NORM_NONE>(a, st);
    case SQ_NORM_LAYERNORM: return dispatch_cfg<CAL, T, SQ_NORM_LAYERNORM>(a, st);
    case SQ_NORM_RMSNORM: return dispatch_cfg<CAL, T, SQ_NORM_RMSNORM>(a, st);
  }
  return hipErrorInvalidValue;
}

template <bool CAL>
hipError_t dispatch_dtype(const RowArgs& a, hipStream_t st) {
  switch (a.dtype) {
    case SQ_DT_F32: return dispatch_norm<CAL, f32_t>(a, st);
    case SQ_DT_F16: return dispatch_norm<CAL, f16_t>(a, st);
    case SQ_DT_BF16: return dispatch_norm<CAL, bf16_t>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_norm_quant(const RowArgs& a, hipStream_t st) { return dispatch_dtype<false>(a, st); }

hipError_t launch_calibrate(const RowArgs& a, hipStream_t st) { return dispatch_dtype<true>(a, st); }

hipError_t launch_fold_colmax_scales(const FoldArgs& f, hipStream_t st) {
  const int K = static_cast<int>(f.K);
  hipLaunchKernelGGL(k_fill_zero, dim3((K + 255) / 256), dim3(256), 0, st, f.s_out, K);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int rows = 256;                                   // keep gridDim.y within 65535
  while ((f.N + rows - 1) / rows > 65535) rows *= 2;
  const dim3 grid(((K >> 3) + 255) / 256, static_cast<unsigned>((f.N + rows - 1) / rows));
  const int N = static_cast<int>(f.N);
  switch (f.dtype) {
    case SQ_DT_F32: hipLaunchKernelGGL(k_colmax<f32_t>, grid, dim3(256), 0, st, f.w, N, K, rows, f.s_out); break;
    case SQ_DT_F16: hipLaunchKernelGGL(k_colmax<f16_t>, grid, dim3(256), 0, st, f.w, N, K, rows, f.s_out); break;
    case SQ_DT_BF16: hipLaunchKernelGGL(k_colmax<bf16_t>, grid, dim3(256), 0, st, f.w, N, K, rows, f.s_out); break;
    default: return hipErrorInvalidValue;
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_scales, dim3((K + 255) / 256), dim3(256), 0, st, f.act_absmax, f.s_out, K, f.alpha,
                     f.eps, f.gamma, f.beta, f.gamma_out, f.beta_out);
  return hipGetLastError();
}

}  // namespace sq
