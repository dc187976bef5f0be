// Row-streaming kernels: fused norm + per-token INT8 quantisation, calibration
// absmax, and the offline fold (weight column maxima, smoothing factors; the
// weight codes are the NONE-norm quantiser run over W with gamma = s).
//
// The quantiser keeps a whole row in registers between its statistics, its
// normalisation and its codes, so each element is read from HBM once and its
// code written once. Workgroups stride over rows and load the next row while
// they work on the current one, which hides HBM latency even when only one
// workgroup fits on a CU (a 20480-wide binary32 row is 80 KiB of registers).
#include "sq_device.h"
#include "sq_launch.h"
#include "smoothquant.h"

namespace sq {

// A row held as raw 16-byte vectors: thread t owns vectors t, t + THREADS, ...
template <typename T, int NV, int THREADS>
struct RawRow {
  Raw8<T> r[NV];
  __device__ __forceinline__ void load(const void* x, int64_t row, int K) {
    const char* xrow = static_cast<const char*>(x) + row * K * Storage<T>::kBytes;
    const int nvec = K >> 3;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int vi = threadIdx.x + i * THREADS;
      if (vi < nvec) raw_load<T>(xrow + static_cast<size_t>(vi) * 8 * Storage<T>::kBytes, r[i]);
      else r[i] = Raw8<T>{};   // padding: zeros, never reloaded
    }
  }
};

// Stand-ins for a missing gamma (ones) or beta (zeros): read at offset 0 for
// every vector, so one code path serves all cases. x * 1 is exact, and x + 0
// differs from x only for -0, which leaves every code and the row maximum as
// they are.
static __constant__ float kOnes8[8] = {1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f};
static __constant__ float kZeros8[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};

// Statistics of a binary32 row held in registers (padding holds zeros) and the
// normalised y in place: LayerNorm ((x - mean) * rstd) * gamma + beta, RMSNorm
// (x * rstd) * gamma; a NULL gamma / beta means 1 / 0. Sums are taken in
// binary64 in a fixed order and rounded once to binary32 (LayerNorm: the
// variance in one pass where that is provably accurate enough, else centred on
// the binary64 mean); rstd = fl32(1 / fl32(sqrt(fl32(var + eps)))).
template <int NORM, int NV, int THREADS>
__device__ __forceinline__ void normalize_row(float (&v)[NV][8], int K, const float* __restrict__ gamma,
                                              const float* __restrict__ beta, float eps, RedRing<THREADS>& red,
                                              int& rk) {
  const int nvec = K >> 3;
  float mu = 0.0f, r = 1.0f;
  if constexpr (NORM == SQ_NORM_LAYERNORM) {
    // One pass: S1 = sum x and S2' = sum x^2 (per-vector partial sums,
    // independent dependency chains, combined in a fixed order), then
    // sum (x - mean)^2 = S2' - S1 * mean. Every x^2 is exact in binary64 and
    // the sums have at most ~24 rounding steps in a chain, so that difference
    // is within 2^-46.7 S2' of the exact value; where S2' <= 256 sum (x - mean)^2
    // this is 2^-38.7 relative, far inside the near-tie margin of the binary32
    // result. Rows whose mean dominates their spread (including constant rows)
    // take the centred second pass instead.
    double p1[NV], q1[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const double d0 = static_cast<double>(v[i][0]);
      p1[i] = d0;
      q1[i] = d0 * d0;
#pragma unroll
      for (int e = 1; e < 8; ++e) {
        const double d = static_cast<double>(v[i][e]);
        p1[i] += d;
        q1[i] = __builtin_fma(d, d, q1[i]);
      }
    }
    double s1 = 0.0, sq = 0.0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      s1 += p1[i];
      sq += q1[i];
    }
    block_sum2<THREADS>(s1, sq, red.at(rk++));
    const double mean = s1 / static_cast<double>(K);
    const double cross = s1 * mean;
    double s2;
    if (cross <= sq * (1.0 - 1.0 / 256.0)) {                 // workgroup-uniform
      s2 = sq - cross;
    } else {
#pragma unroll
      for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) opaque(v[i][e]);   // convert again below rather than keep 2*8*NV doubles
      double p2[NV];
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        p2[i] = 0.0;
        if (static_cast<int>(threadIdx.x) + i * THREADS < nvec) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const double d = static_cast<double>(v[i][e]) - mean;
            p2[i] = __builtin_fma(d, d, p2[i]);
          }
        }
      }
      s2 = 0.0;
#pragma unroll
      for (int i = 0; i < NV; ++i) s2 += p2[i];
      s2 = block_sum<THREADS>(s2, red.at(rk++));
    }
    mu = static_cast<float>(mean);
    r = div_rn(1.0f, sqrt_rn(add_rn(static_cast<float>(s2 / static_cast<double>(K)), eps)));
  } else if constexpr (NORM == SQ_NORM_RMSNORM) {
    double p2[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      p2[i] = 0.0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double d = static_cast<double>(v[i][e]);
        p2[i] = __builtin_fma(d, d, p2[i]);
      }
    }
    double s2 = 0.0;
#pragma unroll
    for (int i = 0; i < NV; ++i) s2 += p2[i];
    s2 = block_sum<THREADS>(s2, red.at(rk++));
    r = div_rn(1.0f, sqrt_rn(add_rn(static_cast<float>(s2 / static_cast<double>(K)), eps)));
  }
  const float* gp = gamma ? gamma : kOnes8;
  const float* bp = beta ? beta : kZeros8;
  const int gmask = gamma ? -1 : 0, bmask = beta ? -1 : 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int vi = threadIdx.x + i * THREADS;
    if (vi >= nvec) continue;
    float g[8], b[8];
    load8_f32(gp + (8 * vi & gmask), g);
    if constexpr (NORM == SQ_NORM_LAYERNORM) load8_f32(bp + (8 * vi & bmask), b);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float t = v[i][e];
      if constexpr (NORM == SQ_NORM_LAYERNORM) t = add_rn(mul_rn(mul_rn(sub_rn(t, mu), r), g[e]), b[e]);
      if constexpr (NORM == SQ_NORM_RMSNORM) t = mul_rn(mul_rn(t, r), g[e]);
      v[i][e] = t;
    }
  }
}

// The per-column factors of the thread's own columns (vectors t, t + THREADS,
// ...), kept for the workgroup's lifetime: a row quantiser reads them for
// every element of every row, twice, which from L2 costs four times the HBM
// bytes of a 16-bit row. Vectors [0, GREG) stay in registers, [GREG, GREG +
// GLDS) in LDS (each thread reads back only what it wrote, so no barrier is
// involved), the rest are re-read from memory.
template <int NV, int THREADS, int GREG, int GLDS>
struct ColVec {
  static_assert(GREG + GLDS <= NV, "column vector split");
  float r[GREG > 0 ? GREG : 1][8];
  float4* lds;                                  // [GLDS][2][THREADS]
  const float* __restrict__ g;
  __device__ __forceinline__ void init(const float* __restrict__ gamma, int nvec, float4* lds_mem) {
    g = gamma;
    lds = lds_mem;
    if (!gamma) return;
#pragma unroll
    for (int i = 0; i < GREG + GLDS; ++i) {
      const int vi = threadIdx.x + i * THREADS;
      float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (vi < nvec) load8_f32(gamma + 8 * vi, v);
      if (i < GREG) {
#pragma unroll
        for (int e = 0; e < 8; ++e) r[i < GREG ? i : 0][e] = v[e];
      } else {
        lds[(2 * (i - GREG)) * THREADS + threadIdx.x] = make_float4(v[0], v[1], v[2], v[3]);
        lds[(2 * (i - GREG) + 1) * THREADS + threadIdx.x] = make_float4(v[4], v[5], v[6], v[7]);
      }
    }
  }
  // factors of vector i (a compile-time index after unrolling)
  __device__ __forceinline__ void get(int i, float v[8]) const {
    if (i < GREG) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = r[i < GREG ? i : 0][e];
    } else if (i < GREG + GLDS) {
      const float4 a = lds[(2 * (i - GREG)) * THREADS + threadIdx.x];
      const float4 b = lds[(2 * (i - GREG) + 1) * THREADS + threadIdx.x];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
      load8_f32(g + 8 * (threadIdx.x + i * THREADS), v);
    }
  }
};

// Split of the column factors for a row layout: as many vectors in registers
// as fit beside the raw row within 128 VGPRs (two 512-thread or one
// 1024-thread workgroup per CU; the rest of the quantiser takes about
// 48 + NV), then LDS up to the workgroup's share (32 / 64 / 128 KiB for
// 256 / 512 / 1024 threads), then memory.
template <typename T, int NV, int THREADS>
struct ColSplit {
  // the wide NONE layout (512 threads, more than 6 vectors each) runs one
  // workgroup per CU: 256 VGPRs per thread and 144 KiB of LDS
  static constexpr bool kWide = THREADS == 512 && NV > 6;
  static constexpr int kBudget = kWide ? 256 : 128;
  static constexpr int kRaw = NV * 2 * Storage<T>::kBytes;
  static constexpr int kFree = (kBudget - kRaw - 48 - NV) / 8;
  static constexpr int kReg = kFree < 0 ? 0 : (kFree < NV ? kFree : NV);
  static constexpr int kLdsCap =
      (kWide ? 147456 : THREADS >= 1024 ? 131072 : THREADS >= 512 ? 65536 : 32768) / (THREADS * 32);
  static constexpr int kLds = NV - kReg < kLdsCap ? NV - kReg : kLdsCap;
};

// y of vector i of a raw row for the NONE norm: x, or fl32(x * gamma).
template <typename T, int NV, int THREADS, int GREG, int GLDS>
__device__ __forceinline__ void none_y(const RawRow<T, NV, THREADS>& raw, int i,
                                       const ColVec<NV, THREADS, GREG, GLDS>& gv, float y[8]) {
  widen8<T>(raw.r[i], y);
  if (gv.g) {
    float g[8];
    gv.get(i, g);
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = mul_rn(y[e], g[e]);
  }
}

// Quantise one row held raw in registers, write its codes and step, and refill
// the raw buffer with row `next` (if next < M) as soon as each part of it is
// free, so the next row's loads overlap this row's work within one buffer.
//  NONE: two passes over the row (the max of |x * gamma|, then the codes).
//        Narrow rows keep the binary32 products and refill the whole buffer
//        before the reduction; wide rows recompute the product in pass two
//        and refill vector i right after its codes are written.
//  LayerNorm / RMSNorm: widen once (the whole buffer is then refilled),
//        normalise in place, then max and codes.
template <typename T, int NORM, int NV, int THREADS, int GREG, int GLDS>
__device__ __forceinline__ void quantize_row(RawRow<T, NV, THREADS>& raw, const void* __restrict__ x,
                                             int64_t row, int64_t next, int M, int K,
                                             const float* __restrict__ gamma,
                                             const ColVec<NV, THREADS, GREG, GLDS>& gv,
                                             const float* __restrict__ beta, float eps, int8_t* __restrict__ xq,
                                             float* __restrict__ x_scale, RedRing<THREADS>& red, int& rk) {
  const int nvec = K >> 3;
  constexpr int B = Storage<T>::kBytes;
  int8_t* qrow = xq + row * K;
  const bool refill = next < M;
  // Address of the next row, formed unconditionally and used only when
  // refill holds. (Written as refill ? next : row, ROCm 7.2's compiler turns
  // the select into an s_cselect on a stale SCC -- the 64-bit compare went to
  // VCC -- and reloads the current row.)
  const char* nrow = static_cast<const char*>(x) + next * K * B;
  if constexpr (NORM == SQ_NORM_NONE) {
    // Narrow rows at up to 512 threads keep pass one's products for pass two
    // (8 NV VGPRs, within the 128 of two workgroups per CU) and refill the raw
    // buffer before the reduction; wider ones recompute x * gamma in pass two.
    constexpr bool kKeepY = THREADS <= 512 && Storage<T>::kBytes == 2 && NV <= 5;
    float ys[kKeepY ? NV : 1][8];
    float pm[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      pm[i] = 0.0f;
      if (static_cast<int>(threadIdx.x) + i * THREADS < nvec) {
        float y[8];
        none_y(raw, i, gv, y);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pm[i] = fmaxf(pm[i], fabsf(y[e]));
          if constexpr (kKeepY) ys[i][e] = y[e];
        }
      }
    }
    if constexpr (kKeepY) {
      if (refill) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          const int vi = threadIdx.x + i * THREADS;
          if (vi < nvec) raw_load<T>(nrow + static_cast<size_t>(vi) * 8 * B, raw.r[i]);
        }
      }
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i) amax = fmaxf(amax, pm[i]);
    amax = block_max<THREADS>(amax, reinterpret_cast<float*>(red.at(rk++)));
    const float step = int8_step(amax);
    if (threadIdx.x == 0) x_scale[row] = step;
    const Quantizer qz(step);
    if constexpr (kKeepY) {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int vi = threadIdx.x + i * THREADS;
        if (vi < nvec) store_codes8(qrow + static_cast<size_t>(vi) * 8, qz.codes8(ys[i]));
      }
    } else {
      // recompute x * gamma below rather than keep pass one's 8*NV products in registers
#pragma unroll
      for (int i = 0; i < NV; ++i) opaque(raw.r[i].a);
      memory_opaque();
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int vi = threadIdx.x + i * THREADS;
        if (vi < nvec) {
          float y[8];
          none_y(raw, i, gv, y);
          store_codes8(qrow + static_cast<size_t>(vi) * 8, qz.codes8(y));
          if (refill) raw_load<T>(nrow + static_cast<size_t>(vi) * 8 * B, raw.r[i]);
        }
      }
    }
  } else {
    float v[NV][8];
#pragma unroll
    for (int i = 0; i < NV; ++i) widen8<T>(raw.r[i], v[i]);   // padding vectors hold zeros
    if (refill) {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int vi = threadIdx.x + i * THREADS;
        if (vi < nvec) raw_load<T>(nrow + static_cast<size_t>(vi) * 8 * B, raw.r[i]);
      }
    }
    normalize_row<NORM, NV, THREADS>(v, K, gamma, beta, eps, red, rk);
    float pm[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      pm[i] = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) pm[i] = fmaxf(pm[i], fabsf(v[i][e]));
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i) amax = fmaxf(amax, pm[i]);
    amax = block_max<THREADS>(amax, reinterpret_cast<float*>(red.at(rk++)));
    const float step = int8_step(amax);
    if (threadIdx.x == 0) x_scale[row] = step;
    const Quantizer qz(step);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int vi = threadIdx.x + i * THREADS;
      if (vi < nvec) store_codes8(qrow + static_cast<size_t>(vi) * 8, qz.codes8(v[i]));
    }
  }
}

// Fused norm + per-token quantisation. Workgroup b handles rows b, b + G, ...
// (G = gridDim.x <= M); one raw row buffer, refilled with the next row while
// the current one is being processed.
template <typename T, int NORM, int NV, int THREADS>
__global__ __launch_bounds__(THREADS) void k_norm_quant(const void* __restrict__ x, int M, int K,
                                                        const float* __restrict__ gamma,
                                                        const float* __restrict__ beta, float eps,
                                                        int8_t* __restrict__ xq, float* __restrict__ x_scale) {
  __shared__ RedRing<THREADS> red;
  // NONE keeps its column factors for the workgroup's lifetime (the norms read
  // gamma / beta once per row)
  constexpr int kReg = NORM == SQ_NORM_NONE ? ColSplit<T, NV, THREADS>::kReg : 0;
  constexpr int kLds = NORM == SQ_NORM_NONE ? ColSplit<T, NV, THREADS>::kLds : 0;
  __shared__ float4 gl[kLds > 0 ? 2 * kLds * THREADS : 1];
  ColVec<NV, THREADS, kReg, kLds> gv;
  const int64_t G = gridDim.x;
  RawRow<T, NV, THREADS> raw;
  raw.load(x, blockIdx.x, K);
  gv.init(NORM == SQ_NORM_NONE ? gamma : nullptr, K >> 3, gl);
  int rk = 0;
  for (int64_t row = blockIdx.x; row < M; row += G)
    quantize_row<T, NORM, NV, THREADS>(raw, x, row, row + G, M, K, gamma, gv, beta, eps, xq, x_scale, red, rk);
}

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
  const int nvec = K >> 3;
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
// 8 in flight (streaming, non-temporal loads); the workgroup then transposes
// its maxima through LDS so that each atomic instruction covers 64 adjacent
// columns (2 cache lines instead of 16), and merges them by atomic max.
// (Workgroups that walk whole rows instead were measured slower: 3.9 against
// 5.6 TB/s on 81920 x 20480.)
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
    for (; r + 8 <= r1; r += 8) {
      Raw8<T> v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const u32x4_t* p = reinterpret_cast<const u32x4_t*>(base + (r + u) * K * B);
        v[u].a = __builtin_bit_cast(uint4, __builtin_nontemporal_load(p));
        if constexpr (B == 4) v[u].b = __builtin_bit_cast(uint4, __builtin_nontemporal_load(p + 1));
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
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

struct RowCfg { int threads, nv; };

// Smallest (threads, vectors per thread) covering K/8 vectors of the row. The
// NONE quantiser of 16-bit rows of 65544 .. 81920 columns takes 512 threads x
// 20 vectors instead of 1024 x 10: one workgroup per CU then holds all of its
// column factors (13 vectors in registers, 7 in LDS) where the 1024-thread
// layout has room for 7 of 10.
RowCfg row_cfg(int K, int norm, int bytes) {
  const int nvec = K >> 3;
  if (norm == SQ_NORM_NONE && bytes == 2 && nvec > 8192 && nvec <= 10240) return {512, 20};
  static const RowCfg table[] = {{256, 1}, {256, 2}, {256, 3}, {256, 4}, {512, 3},  {512, 4},   {512, 5},
                                 {512, 6}, {1024, 4}, {1024, 6}, {1024, 8}, {1024, 10}, {1024, 13}, {1024, 17}};
  for (const RowCfg& c : table)
    if (c.threads * c.nv >= nvec) return c;
  return {1024, 17};
}

// Workgroups that fit on the device at once (all CUs x the kernel's occupancy).
hipError_t resident_blocks(const void* kernel, int threads, int* out) {
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0);
  *out = (e == hipSuccess) ? cus * (per_cu > 0 ? per_cu : 1) : 0;
  return e;
}

template <typename T, int NORM, int NV, int THREADS>
hipError_t launch_nq(const RowArgs& a, hipStream_t st) {
  auto kern = k_norm_quant<T, NORM, NV, THREADS>;
  int cap = 0;
  if (hipError_t e = resident_blocks(reinterpret_cast<const void*>(kern), THREADS, &cap)) return e;
  const int grid = static_cast<int>(a.rows < cap ? a.rows : cap);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(THREADS), 0, st, a.x, static_cast<int>(a.rows), a.K, a.gamma, a.beta,
                     a.eps, a.xq, a.x_scale);
  return hipGetLastError();
}

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
  const int64_t target = 2 * static_cast<int64_t>(cus > 0 ? cus : 256);
  const int64_t row_blocks = (target + col_blocks - 1) / col_blocks;
  int64_t rows = (N + row_blocks - 1) / row_blocks;
  rows = rows < 8 ? 8 : (rows + 7) / 8 * 8;
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

template <bool CAL, typename T, int NORM, int NV, int THREADS>
hipError_t dispatch_one(const RowArgs& a, hipStream_t st) {
  if constexpr (CAL) return launch_cal<T, NORM, NV, THREADS>(a, st);
  else return launch_nq<T, NORM, NV, THREADS>(a, st);
}

template <bool CAL, typename T, int NORM>
hipError_t dispatch_cfg(const RowArgs& a, hipStream_t st) {
  const RowCfg c = row_cfg(a.K, NORM, Storage<T>::kBytes);
  if constexpr (!CAL && NORM == SQ_NORM_NONE && Storage<T>::kBytes == 2) {
    if (c.threads == 512 && c.nv == 20) return dispatch_one<CAL, T, NORM, 20, 512>(a, st);
  }
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
