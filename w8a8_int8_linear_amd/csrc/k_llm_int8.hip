// The LLM.int8() mixed-precision decomposition ("LLM.int8() and SmoothQuant",
// section "Fix 1: give the outliers their own lane (LLM.int8())" and "going
// deeper / LLM.int8() decomposition"): the input channels whose largest
// magnitude over the call's tokens reaches tau are multiplied in 16-bit, the
// rest in INT8 with one step per token and one per output channel, and the two
// products are added. "SmoothQuant, in depth" ("The problem SmoothQuant
// solves") names what this costs at run time: a gather, a second GEMM and a
// merge. Here that is, on the caller's stream:
//
//   1. absmax[j] = max_t |y_tj| over the call's tokens (the calibration
//      kernels: y is the norm output with the model's own gamma, beta);
//   2. k_outlier_select: O = {j : absmax[j] >= tau} as an ascending index
//      list and its count, and gamma, beta with the channels of O zeroed;
//   3. the fused norm + per-token quantiser with those masked parameters: the
//      channels of O come out as exact zeros, so they take code 0 and leave
//      the row's step to the other channels; the norm's (mean, rstd) per row
//      are written out as well;
//   4. k_outlier_gather: the 16-bit operands X[:, O] (y rebuilt from x and the
//      row's mean and rstd with the same binary32 steps, then rounded) and
//      W[:, O], K-contiguous, zero-padded to a multiple of 32;
//   5. the INT8 GEMM with its dequantising epilogue into binary32 (deq);
//   6. k_outlier_merge: acc16 = X[:, O] W[:, O]^T on the 16-bit matrix cores
//      (binary32 accumulation), then out = cvt(fl32(deq + acc16) (+ bias)).
//
// The outlier count lives in device memory only: the host never waits for it.
// Steps 4 and 6 read it and loop over the padded width.
#include "rows.h"

namespace sq {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f_t __attribute__((ext_vector_type(4)));

__global__ void k_fill_zero_f32(float* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

// ----------------------------------------------------------------------------- 2. outlier channels

// One workgroup. Thread t owns the contiguous channels [t c, t c + c), c =
// ceil(K / 1024): it counts its outliers, one workgroup scan gives every
// thread the position of its first one in the ascending list, and a second
// pass over the same channels writes the indices and the masked parameters.
// gamma NULL means 1, beta NULL means 0; beta_m is written only when given.
__global__ __launch_bounds__(1024) void k_outlier_select(const float* __restrict__ absmax, int K, float tau,
                                                         const float* __restrict__ gamma,
                                                         const float* __restrict__ beta, int* __restrict__ count,
                                                         int* __restrict__ idx, float* __restrict__ gamma_m,
                                                         float* __restrict__ beta_m) {
  __shared__ int wsum[1024 / kWave];
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  const int c = (K + 1023) / 1024;
  const int j0 = min(t * c, K), j1 = min(j0 + c, K);
  int n = 0;
  for (int j = j0; j < j1; ++j) n += absmax[j] >= tau ? 1 : 0;
  // inclusive scan inside the wave, then over the wave totals
  int incl = n;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int v = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += v;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int w = 0; w < 1024 / kWave; ++w) {
    base += w < wave ? wsum[w] : 0;
    total += wsum[w];
  }
  int pos = base + incl - n;
  for (int j = j0; j < j1; ++j) {
    const bool o = absmax[j] >= tau;
    if (o) idx[pos++] = j;
    gamma_m[j] = o ? 0.0f : (gamma ? gamma[j] : 1.0f);
    if (beta_m) beta_m[j] = o ? 0.0f : beta[j];
  }
  if (t == 0) *count = total;
}

// ----------------------------------------------------------------------------- 4. 16-bit operands

template <typename T> __device__ __forceinline__ float load1(const void* p, int64_t i);
template <> __device__ __forceinline__ float load1<f32_t>(const void* p, int64_t i) {
  return static_cast<const float*>(p)[i];
}
template <> __device__ __forceinline__ float load1<f16_t>(const void* p, int64_t i) {
  return f16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
}
template <> __device__ __forceinline__ float load1<bf16_t>(const void* p, int64_t i) {
  return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16);
}

// Padded width of the 16-bit operands for `count` outlier channels.
__device__ __forceinline__ int outlier_width(int count) { return (count + 31) & ~31; }

// Rows [0, M) of the grid build X16[m, i], rows [M, M + N) build W16[n, i],
// for i < the padded width (zeros past the count); four rows per workgroup,
// one wave each. y follows the quantiser's binary32 steps: LayerNorm
// fl32(fl32(fl32(x - mean) rstd) gamma) + beta, RMSNorm fl32(fl32(x rstd)
// gamma), a missing gamma or beta skipped; no norm: x. BF16 picks bfloat16,
// else fp16, round half to even.
template <typename TX, typename TW, int NORM, bool BF16>
__global__ __launch_bounds__(256) void k_outlier_gather(const void* __restrict__ x, int M, int K,
                                                        const float* __restrict__ gamma,
                                                        const float* __restrict__ beta,
                                                        const float* __restrict__ stats, const void* __restrict__ w,
                                                        int N, const int* __restrict__ count_p,
                                                        const int* __restrict__ idx, uint16_t* __restrict__ x16,
                                                        uint16_t* __restrict__ w16) {
  const int count = *count_p;
  const int kp = outlier_width(count);
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x / kWave);
  if (row >= static_cast<int64_t>(M) + N) return;
  const bool act = row < M;
  float mu = 0.0f, r = 1.0f;
  if (act && NORM != SQ_NORM_NONE) {
    mu = stats[2 * row];
    r = stats[2 * row + 1];
  }
  uint16_t* dst = act ? x16 + row * kp : w16 + (row - M) * kp;
  for (int i = lane; i < kp; i += kWave) {
    uint32_t h = 0;
    if (i < count) {
      const int j = idx[i];
      float v;
      if (act) {
        v = load1<TX>(x, row * K + j);
        if constexpr (NORM == SQ_NORM_LAYERNORM) {
          v = mul_rn(sub_rn(v, mu), r);
          if (gamma) v = mul_rn(v, gamma[j]);
          if (beta) v = add_rn(v, beta[j]);
        } else if constexpr (NORM == SQ_NORM_RMSNORM) {
          v = mul_rn(v, r);
          if (gamma) v = mul_rn(v, gamma[j]);
        }
      } else {
        v = load1<TW>(w, (row - M) * K + j);
      }
      h = BF16 ? f32_to_bf16_rne(v) : f32_to_f16_rne(v);
    }
    dst[i] = static_cast<uint16_t>(h);
  }
}

// ----------------------------------------------------------------------------- 6. 16-bit product and merge

// One workgroup of four waves per 64 tokens x 128 output channels; wave v takes
// tokens 16 v .. 16 v + 15 against all 128 channels (eight 16 x 16 tiles). The
// matrix-core operand A carries 16 rows of W16 and B 16 rows of X16, each lane
// 8 consecutive K values (lane group g: K offsets 8 g .. 8 g + 7 of the
// 32-wide step, the same for both operands), so lane l ends with acc16 of
// token l % 16 and the four consecutive channels 4 (l / 16) .. + 3 of a tile.
// The merge then reads those four deq values with one 16-byte load.
template <int YDT, bool BF16>
__global__ __launch_bounds__(256) void k_outlier_merge(const uint16_t* __restrict__ x16,
                                                       const uint16_t* __restrict__ w16,
                                                       const int* __restrict__ count_p,
                                                       const float* __restrict__ deq,
                                                       const float* __restrict__ bias, void* __restrict__ y, int M,
                                                       int N) {
  constexpr int TJ16 = 8;
  const int kp = outlier_width(*count_p);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int r16 = lane & 15, g = lane >> 4;
  const int m0 = blockIdx.y * 64 + 16 * wave, n0 = blockIdx.x * 128;
  v4f_t acc[TJ16];
#pragma unroll
  for (int j = 0; j < TJ16; ++j) acc[j] = v4f_t{0.0f, 0.0f, 0.0f, 0.0f};
  const int64_t xrow = min(m0 + r16, M - 1);
  for (int k0 = 0; k0 < kp; k0 += 32) {
    const uint4 bx = *reinterpret_cast<const uint4*>(x16 + xrow * kp + k0 + 8 * g);
#pragma unroll
    for (int j = 0; j < TJ16; ++j) {
      const int64_t wrow = min(n0 + 16 * j + r16, N - 1);
      const uint4 aw = *reinterpret_cast<const uint4*>(w16 + wrow * kp + k0 + 8 * g);
      if constexpr (BF16)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, aw), __builtin_bit_cast(v8bf, bx),
                                                         acc[j], 0, 0, 0);
      else
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, aw), __builtin_bit_cast(v8h, bx),
                                                        acc[j], 0, 0, 0);
    }
  }
  const int m = m0 + r16;
  if (m >= M) return;
  const bool vec = (N & 3) == 0;
#pragma unroll
  for (int j = 0; j < TJ16; ++j) {
    const int n = n0 + 16 * j + 4 * g;
    if (n >= N) continue;
    const int64_t off = static_cast<int64_t>(m) * N + n;
    const bool full = vec && n + 3 < N;
    float d[4], o[4];
    if (full) {
      const float4 q = *reinterpret_cast<const float4*>(deq + off);
      d[0] = q.x; d[1] = q.y; d[2] = q.z; d[3] = q.w;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) d[r] = n + r < N ? deq[off + r] : 0.0f;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float t = add_rn(d[r], acc[j][r]);
      if (bias) t = add_rn(t, bias[min(n + r, N - 1)]);
      o[r] = t;
    }
    if constexpr (YDT == SQ_DT_F32) {
      float* p = static_cast<float*>(y) + off;
      if (full) {
        *reinterpret_cast<float4*>(p) = make_float4(o[0], o[1], o[2], o[3]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (n + r < N) p[r] = o[r];
      }
    } else {
      uint32_t h[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) h[r] = YDT == SQ_DT_F16 ? f32_to_f16_rne(o[r]) : f32_to_bf16_rne(o[r]);
      uint16_t* p = static_cast<uint16_t*>(y) + off;
      if (full) {
        *reinterpret_cast<uint2*>(p) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (n + r < N) p[r] = static_cast<uint16_t>(h[r]);
      }
    }
  }
}

// ----------------------------------------------------------------------------- launchers

namespace {

template <typename T, int NORM>
struct StatsLaunch {
  const RowArgs& a;
  hipStream_t st;
  template <int NV, int THREADS>
  hipError_t run() const { return launch_nq<T, NORM, NV, THREADS, kRowsStats>(a, nullptr, 0, st); }
};

template <typename T>
hipError_t launch_stats_t(const RowArgs& a, hipStream_t st) {
  constexpr int B = Storage<T>::kBytes;
  if (a.norm == SQ_NORM_LAYERNORM)
    return with_row_cfg<false>(a.K, SQ_NORM_LAYERNORM, B, StatsLaunch<T, SQ_NORM_LAYERNORM>{a, st});
  if (a.norm == SQ_NORM_RMSNORM)
    return with_row_cfg<false>(a.K, SQ_NORM_RMSNORM, B, StatsLaunch<T, SQ_NORM_RMSNORM>{a, st});
  return hipErrorInvalidValue;
}

template <typename TX, typename TW, int NORM>
hipError_t launch_gather_t(const LlmArgs& l, hipStream_t st) {
  const int64_t rows = l.M + l.N;
  const dim3 grid(static_cast<unsigned>((rows + 3) / 4));
  if (std::is_same<TW, bf16_t>::value)
    hipLaunchKernelGGL((k_outlier_gather<TX, TW, NORM, true>), grid, dim3(256), 0, st, l.x, l.M, l.K, l.gamma, l.beta,
                       l.stats, l.w, l.N, l.count, l.idx, l.x16, l.w16);
  else
    hipLaunchKernelGGL((k_outlier_gather<TX, TW, NORM, false>), grid, dim3(256), 0, st, l.x, l.M, l.K, l.gamma,
                       l.beta, l.stats, l.w, l.N, l.count, l.idx, l.x16, l.w16);
  return hipGetLastError();
}

template <typename TX, typename TW>
hipError_t launch_gather_n(const LlmArgs& l, hipStream_t st) {
  switch (l.norm) {
    case SQ_NORM_NONE: return launch_gather_t<TX, TW, SQ_NORM_NONE>(l, st);
    case SQ_NORM_LAYERNORM: return launch_gather_t<TX, TW, SQ_NORM_LAYERNORM>(l, st);
    case SQ_NORM_RMSNORM: return launch_gather_t<TX, TW, SQ_NORM_RMSNORM>(l, st);
  }
  return hipErrorInvalidValue;
}

template <typename TX>
hipError_t launch_gather_w(const LlmArgs& l, hipStream_t st) {
  switch (l.w_dt) {
    case SQ_DT_F32: return launch_gather_n<TX, f32_t>(l, st);
    case SQ_DT_F16: return launch_gather_n<TX, f16_t>(l, st);
    case SQ_DT_BF16: return launch_gather_n<TX, bf16_t>(l, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gather(const LlmArgs& l, hipStream_t st) {
  switch (l.x_dt) {
    case SQ_DT_F32: return launch_gather_w<f32_t>(l, st);
    case SQ_DT_F16: return launch_gather_w<f16_t>(l, st);
    case SQ_DT_BF16: return launch_gather_w<bf16_t>(l, st);
    default: return hipErrorInvalidValue;
  }
}

template <int YDT>
hipError_t launch_merge_t(const LlmArgs& l, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((l.N + 127) / 128), static_cast<unsigned>((l.M + 63) / 64));
  if (l.w_dt == SQ_DT_BF16)
    hipLaunchKernelGGL((k_outlier_merge<YDT, true>), grid, dim3(256), 0, st, l.x16, l.w16, l.count, l.deq, l.bias,
                       l.y, l.M, l.N);
  else
    hipLaunchKernelGGL((k_outlier_merge<YDT, false>), grid, dim3(256), 0, st, l.x16, l.w16, l.count, l.deq, l.bias,
                       l.y, l.M, l.N);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_llm_int8(const LlmArgs& l, hipStream_t st) {
  hipError_t e;
  // 1. the call's per-channel maxima of the linear's input
  hipLaunchKernelGGL(k_fill_zero_f32, dim3((l.K + 255) / 256), dim3(256), 0, st, l.absmax, l.K);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const RowArgs cal{l.x, l.x_dt, l.M, l.K, l.norm, l.norm == SQ_NORM_NONE ? nullptr : l.gamma,
                    l.norm == SQ_NORM_LAYERNORM ? l.beta : nullptr, l.eps, nullptr, nullptr, l.absmax};
  if ((e = launch_calibrate(cal, st)) != hipSuccess) return e;
  // 2. the outlier channels, and the norm's parameters with them zeroed
  const float* gamma = l.norm == SQ_NORM_NONE ? nullptr : l.gamma;
  const float* beta = l.norm == SQ_NORM_LAYERNORM ? l.beta : nullptr;
  hipLaunchKernelGGL(k_outlier_select, dim3(1), dim3(1024), 0, st, l.absmax, l.K, l.tau, gamma, beta, l.count, l.idx,
                     l.gamma_m, beta ? l.beta_m : nullptr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // 3. INT8 codes of the other channels, one step per token (and the row statistics)
  RowArgs q{l.x, l.x_dt, l.M, l.K, l.norm, l.gamma_m, beta ? l.beta_m : nullptr, l.eps, l.xq, l.x_scale, nullptr};
  if (l.norm == SQ_NORM_NONE) {
    e = launch_norm_quant(q, st);
  } else {
    q.stats = l.stats;
    switch (l.x_dt) {
      case SQ_DT_F32: e = launch_stats_t<f32_t>(q, st); break;
      case SQ_DT_F16: e = launch_stats_t<f16_t>(q, st); break;
      case SQ_DT_BF16: e = launch_stats_t<bf16_t>(q, st); break;
      default: e = hipErrorInvalidValue;
    }
  }
  if (e != hipSuccess) return e;
  // 4. the 16-bit operands of the outlier channels
  LlmArgs g = l;
  g.gamma = gamma;
  g.beta = beta;
  if ((e = launch_gather(g, st)) != hipSuccess) return e;
  // 5. the INT8 product, dequantised into binary32
  const GemmArgs gm{l.xq, l.x_scale, l.wq, l.w_scale, nullptr, l.deq, SQ_DT_F32, static_cast<int>(l.M),
                    static_cast<int>(l.N), l.K};
  if ((e = launch_gemm(gm, st)) != hipSuccess) return e;
  // 6. the 16-bit product, added to it
  switch (l.y_dt) {
    case SQ_DT_F32: return launch_merge_t<SQ_DT_F32>(l, st);
    case SQ_DT_F16: return launch_merge_t<SQ_DT_F16>(l, st);
    case SQ_DT_BF16: return launch_merge_t<SQ_DT_BF16>(l, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sq
