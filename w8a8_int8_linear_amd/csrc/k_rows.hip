// Row-streaming kernels: fused norm + per-token quantisation, calibration
// absmax, and the offline fold (weight column maxima, smoothing factors; the
// weight codes are the NONE-norm quantiser run over W with gamma = s). The
// building blocks they share with the per-tensor passes are in rows.h.
#include "rows.h"

namespace sq {

// Calibration with a norm: workgroups stride over rows, normalise each with the
// unfolded gamma / beta, keep the per-column max of |y| in registers and merge
// it into absmax with an order-free atomic max at the end.
template <typename T, int NORM, int NV, int THREADS>
__global__ __launch_bounds__(THREADS) void k_calibrate(const void* __restrict__ x, int M, int K,
                                                       const float* __restrict__ gamma,
                                                       const float* __restrict__ beta, float eps,
                                                       float* __restrict__ absmax) {
  __shared__ RedRing<THREADS> red;
  __shared__ float4 gl[2 * THREADS];                       // 8 floats per thread: the merge transpose
  int rk = 0;
  float cm[NV][8];
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) cm[i][e] = 0.0f;
  for (int64_t row = blockIdx.x; row < M; row += gridDim.x) {
    RawRow<T, NV, THREADS> raw;
    raw.load(x, row, K);
    float v[NV][8];
#pragma unroll
    for (int i = 0; i < NV; ++i) widen8<T>(raw.r[i], v[i]);   // padding vectors hold zeros
    normalize_row<NORM, NV, THREADS>(v, K, gamma, beta, eps, red, rk);
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) cm[i][e] = fmaxf(cm[i][e], fabsf(v[i][e]));
  }
  // Merge by atomic max after a transpose through LDS: chunk i (columns
  // 8 i THREADS .. +8 THREADS) is written as thread t's 8 columns at 8t, and
  // read back as columns t, t + THREADS, ..., so each atomic instruction
  // covers 64 adjacent columns (2 cache lines instead of 16).
  float* t_lds = reinterpret_cast<float*>(gl);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c0 = 8 * i * THREADS;
    if (c0 >= K) break;                                    // uniform
    __syncthreads();                                       // previous chunk's reads are done
#pragma unroll
    for (int e = 0; e < 8; ++e) t_lds[threadIdx.x * 8 + e] = cm[i][e];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = c0 + threadIdx.x + THREADS * j;
      if (c < K) atomic_max_nonneg(absmax + c, t_lds[threadIdx.x + THREADS * j]);
    }
  }
}

// Column maxima colmax[j] = max(colmax[j], max_n |X[n, j]|): the weight column
// maxima of the fold (colmax pre-zeroed), and calibration without a norm (the
// running absmax). Each thread owns 8 adjacent columns and walks `rows` rows,
// 16 in flight (streaming, non-temporal loads); the workgroup then transposes
// its maxima through LDS so that each atomic instruction covers 64 adjacent
// columns (2 cache lines instead of 16), and merges them by atomic max.
// (Measured on 81920 x 20480 fp16: 16 rows in flight 6.6 TB/s, 8 rows 5.6,
// 32 rows or four workgroups per CU 6.4-6.5; workgroups that walk whole rows
// instead 3.9 TB/s.)
constexpr int kColmaxRows = 16;      // rows in flight per thread
constexpr int kColmaxPerCu = 2;      // workgroups per CU in the grid

template <typename T>
__global__ __launch_bounds__(256) void k_colmax(const void* __restrict__ w, int N, int K, int rows,
                                                float* __restrict__ colmax) {
  __shared__ float t_lds[256 * 8];
  const int vi = blockIdx.x * 256 + threadIdx.x;
  const int nvec = K >> 3;
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * rows;
  const int64_t r1 = r0 + rows < N ? r0 + rows : N;
  constexpr int B = Storage<T>::kBytes;
  float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (vi < nvec) {
    const char* base = static_cast<const char*>(w) + static_cast<size_t>(vi) * 8 * B;
    int64_t r = r0;
    for (; r + kColmaxRows <= r1; r += kColmaxRows) {
      Raw8<T> v[kColmaxRows];
#pragma unroll
      for (int u = 0; u < kColmaxRows; ++u) {
        const u32x4_t* p = reinterpret_cast<const u32x4_t*>(base + (r + u) * K * B);
        v[u].a = __builtin_bit_cast(uint4, __builtin_nontemporal_load(p));
        if constexpr (B == 4) v[u].b = __builtin_bit_cast(uint4, __builtin_nontemporal_load(p + 1));
      }
#pragma unroll
      for (int u = 0; u < kColmaxRows; ++u) {
        float f[8];
        widen8<T>(v[u], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) m[e] = fmaxf(m[e], fabsf(f[e]));
      }
    }
    for (; r < r1; ++r) {
      float f[8];
      load8<T>(base + r * K * B, f);
#pragma unroll
      for (int e = 0; e < 8; ++e) m[e] = fmaxf(m[e], fabsf(f[e]));
    }
  }
  // transpose: thread t holds columns c0 + 8t .. +8; then thread t merges columns c0 + t, c0 + t + 256, ...
#pragma unroll
  for (int e = 0; e < 8; ++e) t_lds[threadIdx.x * 8 + e] = m[e];
  __syncthreads();
  const int c0 = blockIdx.x * 2048;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int c = c0 + threadIdx.x + 256 * j;
    if (c < K) atomic_max_nonneg(colmax + c, t_lds[threadIdx.x + 256 * j]);
  }
}

__global__ void k_fill_zero(float* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

// Smoothing factors: s_j = max(fl32(max(a_j, eps)^alpha / max(w_j, eps)^(1 - alpha)), eps)
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

template <typename T, int NORM, int NV, int THREADS>
hipError_t launch_cal(const RowArgs& a, hipStream_t st) {
  // enough rows per workgroup to keep the atomic merges few, enough workgroups to fill the device
  auto kern = k_calibrate<T, NORM, NV, THREADS>;
  int cap = 0;
  if (hipError_t e = resident_blocks(reinterpret_cast<const void*>(kern), THREADS, &cap)) return e;
  int64_t grid = (a.rows + 3) / 4;
  if (grid > cap) grid = cap;
  hipLaunchKernelGGL(kern, dim3(static_cast<int>(grid)), dim3(THREADS), 0, st, a.x, static_cast<int>(a.rows), a.K,
                     a.gamma, a.beta, a.eps, a.absmax);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_colmax(const void* x, int64_t N, int K, float* colmax, hipStream_t st) {
  // rows per workgroup: about two workgroups per CU in all (each merges 2048
  // columns by atomic max, so fewer, longer workgroups keep the atomics few),
  // a multiple of 8, gridDim.y within 65535
  int cus = 0, dev = 0;
  if (hipError_t e = hipGetDevice(&dev)) return e;
  if (hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) return e;
  const int64_t col_blocks = ((K >> 3) + 255) / 256;
  const int64_t target = kColmaxPerCu * static_cast<int64_t>(cus > 0 ? cus : 256);
  const int64_t row_blocks = (target + col_blocks - 1) / col_blocks;
  int64_t rows = (N + row_blocks - 1) / row_blocks;
  rows = rows < kColmaxRows ? kColmaxRows : (rows + kColmaxRows - 1) / kColmaxRows * kColmaxRows;
  while ((N + rows - 1) / rows > 65535) rows *= 2;
  const dim3 grid(static_cast<unsigned>(col_blocks), static_cast<unsigned>((N + rows - 1) / rows));
  hipLaunchKernelGGL(k_colmax<T>, grid, dim3(256), 0, st, x, static_cast<int>(N), K, static_cast<int>(rows), colmax);
  return hipGetLastError();
}

hipError_t launch_colmax_dt(sq_dtype dt, const void* x, int64_t N, int K, float* colmax, hipStream_t st) {
  switch (dt) {
    case SQ_DT_F32: return launch_colmax<f32_t>(x, N, K, colmax, st);
    case SQ_DT_F16: return launch_colmax<f16_t>(x, N, K, colmax, st);
    case SQ_DT_BF16: return launch_colmax<bf16_t>(x, N, K, colmax, st);
    default: return hipErrorInvalidValue;
  }
}

template <bool CAL, typename T, int NORM>
struct RowLaunch {
  const RowArgs& a;
  hipStream_t st;
  template <int NV, int THREADS>
  hipError_t run() const {
    if constexpr (CAL) return launch_cal<T, NORM, NV, THREADS>(a, st);
    else return launch_nq<T, NORM, NV, THREADS, kRowsPerRow>(a, nullptr, 0, st);
  }
};

template <bool CAL, typename T, int NORM>
hipError_t dispatch_cfg(const RowArgs& a, hipStream_t st) {
  constexpr bool kWide = !CAL && NORM == SQ_NORM_NONE && Storage<T>::kBytes == 2;
  return with_row_cfg<kWide>(a.K, NORM, Storage<T>::kBytes, RowLaunch<CAL, T, NORM>{a, st});
}

template <bool CAL, typename T>
hipError_t dispatch_norm(const RowArgs& a, hipStream_t st) {
  switch (a.norm) {
    case SQ_NORM_NONE:
      if constexpr (CAL) return hipErrorInvalidValue;   // NONE calibration is a column max
      else return dispatch_cfg<CAL, T, SQ_NORM_NONE>(a, st);
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

hipError_t launch_calibrate(const RowArgs& a, hipStream_t st) {
  // Without a norm the linear's input is x itself: the running absmax is a column max.
  if (a.norm == SQ_NORM_NONE) return launch_colmax_dt(a.dtype, a.x, a.rows, a.K, a.absmax, st);
  return dispatch_dtype<true>(a, st);
}

hipError_t launch_fold_colmax_scales(const FoldArgs& f, hipStream_t st) {
  const int K = static_cast<int>(f.K);
  hipLaunchKernelGGL(k_fill_zero, dim3((K + 255) / 256), dim3(256), 0, st, f.s_out, K);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = launch_colmax_dt(f.dtype, f.w, f.N, K, f.s_out, st)) != hipSuccess) return e;
  hipLaunchKernelGGL(k_scales, dim3((K + 255) / 256), dim3(256), 0, st, f.act_absmax, f.s_out, K, f.alpha,
                     f.eps, f.gamma, f.beta, f.gamma_out, f.beta_out);
  return hipGetLastError();
}

}  // namespace sq
