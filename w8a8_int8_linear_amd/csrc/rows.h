// Row-streaming building blocks shared by the row kernels: a row held in
// registers, the norm's statistics and elementwise steps, the per-column
// factors kept on chip, the row quantiser (per-row and per-tensor steps), the
// fused norm + quantise kernel template, and the host-side choice of a row
// layout (threads x 16-byte vectors per thread) for a row length.
//
// The quantiser keeps a whole row in registers between its statistics, its
// normalisation and its codes, so each element is read from HBM once and its
// code written once. Workgroups stride over rows and load the next row while
// they work on the current one, which hides HBM latency even when only one
// workgroup fits on a CU (a 20480-wide binary32 row is 80 KiB of registers).
#pragma once

#include <type_traits>

#include "sq_device.h"
#include "sq_launch.h"
#include "smoothquant.h"

namespace sq {

// A row held as raw 16-byte vectors: thread t owns vectors t, t + THREADS, ...
template <typename T, int NV, int THREADS>
struct RawRow {
  Raw8<T> r[NV];
  // byte offset of the thread's vector i within a row
  static __device__ __forceinline__ uint32_t off(int i) {
    return static_cast<uint32_t>(threadIdx.x + i * THREADS) * (8 * Storage<T>::kBytes);
  }
  // buffer resource of row `row` (uniform)
  static __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* x, int64_t row, int K) {
    return buf_rsrc(static_cast<const char*>(x) + row * K * Storage<T>::kBytes,
                    static_cast<uint32_t>(K) * Storage<T>::kBytes);
  }
  __device__ __forceinline__ void load(const void* x, int64_t row, int K) {
    const __amdgpu_buffer_rsrc_t rr = rsrc(x, row, K);
#pragma unroll
    for (int i = 0; i < NV; ++i) raw_load_buf<T>(rr, off(i), r[i]);   // padding vectors read zeros
  }
};

// Stand-ins for a missing gamma (ones) or beta (zeros): read at offset 0 for
// every vector, so one code path serves all cases. x * 1 is exact, and x + 0
// differs from x only for -0, which leaves every code and the row maximum as
// they are.
static __constant__ float kOnes8[8] = {1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f};
static __constant__ float kZeros8[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};

// On-chip copy of the norm's gamma (and LayerNorm's beta) for the first GB
// vectors of each thread, kept for the workgroup's lifetime: every row reads
// them, and from memory those loads wait, in issue order, behind the next
// row's refill. Each thread reads back only what it wrote (no barrier). GB
// fills a share of LDS that leaves room for the layout's workgroups per CU:
// 32 / 64 / 128 KiB for 256 / 512 / 1024 threads; rows of fewer than 4
// vectors per thread keep GB = 0.
template <int NORM, int GB, int THREADS>
struct NormCache {
  static constexpr int kParts = NORM == SQ_NORM_LAYERNORM ? 2 : 1;   // gamma (and beta)
  static constexpr int kFloat4 = GB > 0 ? GB * kParts * 2 * THREADS : 1;
  static __device__ __forceinline__ void init(float4* c, const float* __restrict__ gamma,
                                              const float* __restrict__ beta, int nvec) {
#pragma unroll
    for (int i = 0; i < GB; ++i) {
      const int vi = threadIdx.x + i * THREADS;
#pragma unroll
      for (int part = 0; part < kParts; ++part) {
        const float* src = part == 0 ? gamma : beta;
        float w[8] = {part == 0 ? 1.0f : 0.0f, part == 0 ? 1.0f : 0.0f, part == 0 ? 1.0f : 0.0f,
                      part == 0 ? 1.0f : 0.0f, part == 0 ? 1.0f : 0.0f, part == 0 ? 1.0f : 0.0f,
                      part == 0 ? 1.0f : 0.0f, part == 0 ? 1.0f : 0.0f};
        if (src != nullptr && vi < nvec) load8_f32(src + 8 * vi, w);
        c[((i * kParts + part) * 2) * THREADS + threadIdx.x] = make_float4(w[0], w[1], w[2], w[3]);
        c[((i * kParts + part) * 2 + 1) * THREADS + threadIdx.x] = make_float4(w[4], w[5], w[6], w[7]);
      }
    }
  }
  static __device__ __forceinline__ void get(const float4* __restrict__ c, int i, float g[8], float b[8]) {
    const float4 g0 = c[((i * kParts) * 2) * THREADS + threadIdx.x];
    const float4 g1 = c[((i * kParts) * 2 + 1) * THREADS + threadIdx.x];
    g[0] = g0.x; g[1] = g0.y; g[2] = g0.z; g[3] = g0.w; g[4] = g1.x; g[5] = g1.y; g[6] = g1.z; g[7] = g1.w;
    if constexpr (kParts == 2) {
      const float4 b0 = c[((i * kParts + 1) * 2) * THREADS + threadIdx.x];
      const float4 b1 = c[((i * kParts + 1) * 2 + 1) * THREADS + threadIdx.x];
      b[0] = b0.x; b[1] = b0.y; b[2] = b0.z; b[3] = b0.w; b[4] = b1.x; b[5] = b1.y; b[6] = b1.z; b[7] = b1.w;
    }
  }
};
template <int NORM, int NV, int THREADS>
constexpr int norm_cache_vectors() {
  if (NORM == SQ_NORM_NONE || NV < 4) return 0;
  const int budget = THREADS >= 1024 ? 131072 : THREADS >= 512 ? 65536 : 32768;
  const int per = (NORM == SQ_NORM_LAYERNORM ? 2 : 1) * 32 * THREADS;
  return budget / per < NV ? budget / per : NV;
}

// Statistics of a binary32 row held in registers (padding holds zeros) and the
// normalised y in place: LayerNorm ((x - mean) * rstd) * gamma + beta, RMSNorm
// (x * rstd) * gamma; a NULL gamma / beta means 1 / 0. Sums are taken in
// binary64 in a fixed order and rounded once to binary32 (LayerNorm: the
// variance in one pass where that is provably accurate enough, else centred on
// the binary64 mean); rstd = fl32(1 / fl32(sqrt(fl32(var + eps)))). With st
// non-NULL, thread 0 also writes (mean, rstd) there (mean 0 for RMSNorm).
// With GB > 0, gamma and beta of the thread's vectors [0, GB) are read from
// gbl, the workgroup's on-chip copy (NormCache below), instead of memory.
template <int NORM, int NV, int THREADS, int GB = 0>
__device__ __forceinline__ void normalize_row(float (&v)[NV][8], int K, const float* __restrict__ gamma,
                                              const float* __restrict__ beta, float eps, RedRing<THREADS>& red,
                                              int& rk, float* __restrict__ st = nullptr,
                                              const float4* __restrict__ gbl = nullptr) {
  const int nvec = K >> 3;
  // 1/K in binary64, the same for every row: a product with it is within 2^-52
  // relative of the quotient, far inside the 2^-12-spacing near-tie margin of
  // the binary32 statistics (a division per row cost two binary64 divide
  // sequences of every wave)
  const double inv_k = 1.0 / static_cast<double>(K);
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
    const double mean = s1 * inv_k;
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
    r = div_rn(1.0f, sqrt_rn(add_rn(static_cast<float>(s2 * inv_k), eps)));
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
    r = div_rn(1.0f, sqrt_rn(add_rn(static_cast<float>(s2 * inv_k), eps)));
  }
  if (st != nullptr && threadIdx.x == 0) {
    st[0] = mu;
    st[1] = r;
  }
  // gamma / beta through buffer resources (uniform) at per-thread offsets that
  // are the same for every row; a missing one reads the stand-in at offset 0
  const __amdgpu_buffer_rsrc_t rg = buf_rsrc(gamma ? gamma : kOnes8, gamma ? 4u * static_cast<uint32_t>(K) : 32u);
  const __amdgpu_buffer_rsrc_t rb = buf_rsrc(beta ? beta : kZeros8, beta ? 4u * static_cast<uint32_t>(K) : 32u);
  const uint32_t gmask = gamma ? ~0u : 0u, bmask = beta ? ~0u : 0u;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int vi = threadIdx.x + i * THREADS;
    if (vi >= nvec) continue;
    float g[8], b[8];
    if (i < GB) {
      NormCache<NORM, GB, THREADS>::get(gbl, i < GB ? i : 0, g, b);
    } else {
      load8_f32_buf(rg, (32u * static_cast<uint32_t>(vi)) & gmask, g);
      if constexpr (NORM == SQ_NORM_LAYERNORM) load8_f32_buf(rb, (32u * static_cast<uint32_t>(vi)) & bmask, b);
    }
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
//        normalise in place, then max and codes; STATS also writes the
//        row's (mean, rstd) to stats[2 row], stats[2 row + 1].
template <typename T, int NORM, int NV, int THREADS, int GREG, int GLDS, bool FP8 = false, bool STATS = false,
          int GB = 0>
__device__ __forceinline__ void quantize_row(RawRow<T, NV, THREADS>& raw, const void* __restrict__ x,
                                             int64_t row, int64_t next, int M, int K,
                                             const float* __restrict__ gamma,
                                             const ColVec<NV, THREADS, GREG, GLDS>& gv,
                                             const float* __restrict__ beta, float eps, int8_t* __restrict__ xq,
                                             float* __restrict__ x_scale, RedRing<THREADS>& red, int& rk,
                                             float* __restrict__ stats = nullptr,
                                             const float4* __restrict__ gbl = nullptr) {
  const int nvec = K >> 3;
  using RR = RawRow<T, NV, THREADS>;
  const __amdgpu_buffer_rsrc_t rq = buf_rsrc(xq + row * K, static_cast<uint32_t>(K));   // this row's codes
  const bool refill = next < M;
  // Resource of the next row, formed unconditionally and used only when
  // refill holds. (Written as refill ? next : row, ROCm 7.2's compiler turns
  // the select into an s_cselect on a stale SCC -- the 64-bit compare went to
  // VCC -- and reloads the current row.)
  const __amdgpu_buffer_rsrc_t rn = RR::rsrc(x, next, K);
  if constexpr (NORM == SQ_NORM_NONE) {
    // Narrow rows at up to 512 threads keep pass one's products for pass two
    // (8 NV VGPRs, within the 128 of two workgroups per CU) and refill the raw
    // buffer before the reduction; wider ones recompute x * gamma in pass two.
    constexpr bool kKeepY = THREADS <= 512 && Storage<T>::kBytes == 2 && NV <= 5;
    // Wide rows with every column factor on chip (padding vectors hold zero
    // factors, and their raw vectors read zeros) run both passes with no
    // per-vector branch: each padding store falls past the codes' K bytes and
    // is dropped. The wait-counter pass then tracks each vector's refill
    // separately, and pass one starts on vector 0 of the next row while later
    // vectors are still in flight. Behind per-vector branches it waited for
    // the whole row first (vmcnt(0)).
    constexpr bool kFlat = !kKeepY && GREG + GLDS == NV;
    float ys[kKeepY ? NV : 1][8];
    float pm[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      pm[i] = 0.0f;
      if (kFlat || static_cast<int>(threadIdx.x) + i * THREADS < nvec) {
        float y[8];
        none_y(raw, i, gv, y);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pm[i] = fmaxf(pm[i], fabsf(y[e]));
          if constexpr (kKeepY) ys[i][e] = y[e];
        }
      }
      if constexpr (kFlat) {
        // one vector at a time, as the branches kept it: each vector's max is
        // formed here rather than in one tree over every vector's products
        asm volatile("" : "+v"(pm[i]));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (kKeepY) {
      if (refill) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          const int vi = threadIdx.x + i * THREADS;
          if (vi < nvec) raw_load_buf<T>(rn, RR::off(i), raw.r[i]);
        }
      }
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i) amax = fmaxf(amax, pm[i]);
    amax = block_max<THREADS>(amax, reinterpret_cast<float*>(red.at(rk++)));
    const float step = FP8 ? fp8_step(amax) : int8_step(amax);
    if (threadIdx.x == 0) x_scale[row] = step;
    const typename std::conditional<FP8, QuantizerFp8, Quantizer>::type qz(step);
    if constexpr (kKeepY) {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int vi = threadIdx.x + i * THREADS;
        if (vi < nvec) store_codes8_buf(rq, static_cast<uint32_t>(vi) * 8, qz.codes8(ys[i]));
      }
    } else {
      // recompute x * gamma below rather than keep pass one's 8*NV products in registers
#pragma unroll
      for (int i = 0; i < NV; ++i) opaque(raw.r[i].a);
      memory_opaque();
      // (kFlat) the vector index base, opaque per row: hoisted out of the row
      // loop, the 2 NV code and refill offsets would each hold a register
      uint32_t ob = threadIdx.x;
      if constexpr (kFlat) asm volatile("" : "+v"(ob));
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int vi = threadIdx.x + i * THREADS;
        if (kFlat || vi < nvec) {
          float y[8];
          none_y(raw, i, gv, y);
          const uint32_t v = kFlat ? ob + static_cast<uint32_t>(i * THREADS) : static_cast<uint32_t>(vi);
          store_codes8_buf(rq, v * 8, qz.codes8(y));
          if (refill) raw_load_buf<T>(rn, kFlat ? v * (8 * Storage<T>::kBytes) : RR::off(i), raw.r[i]);
        }
        if constexpr (kFlat) __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else {
    float v[NV][8];
#pragma unroll
    for (int i = 0; i < NV; ++i) widen8<T>(raw.r[i], v[i]);   // padding vectors hold zeros
    // Rows of 4 or more vectors per thread request every vector (padding
    // reads zeros), with no per-vector branch and no register copies at the
    // loop latch: LayerNorm 8192x20480 ran 1-4% faster. Shorter rows keep the
    // per-vector guard, which measured 1-3% faster on them (2048x4096 LN,
    // 4096x4096 RMSNorm).
    if (refill) {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        if constexpr (NV >= 4) {
          raw_load_buf<T>(rn, RR::off(i), raw.r[i]);
        } else {
          if (static_cast<int>(threadIdx.x) + i * THREADS < nvec) raw_load_buf<T>(rn, RR::off(i), raw.r[i]);
        }
      }
    }
    normalize_row<NORM, NV, THREADS, GB>(v, K, gamma, beta, eps, red, rk, STATS ? stats + 2 * row : nullptr, gbl);
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
    const float step = FP8 ? fp8_step(amax) : int8_step(amax);
    if (threadIdx.x == 0) x_scale[row] = step;
    const typename std::conditional<FP8, QuantizerFp8, Quantizer>::type qz(step);
    // every vector stores (a padding vector's offset lies past the codes' K
    // bytes, so the store is dropped): no per-vector branch
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int vi = threadIdx.x + i * THREADS;
      store_codes8_buf(rq, static_cast<uint32_t>(vi) * 8, qz.codes8(v[i]));
    }
  }
}

// Modes of the fused norm + quantise kernel.
constexpr int kRowsPerRow = 0;       // one step per row (per-token activations, per-channel weights)
constexpr int kRowsAmax = 1;         // per-tensor first pass: each row's max |y| into x_scale[row]; no codes
constexpr int kRowsGivenStep = 2;    // per-tensor codes with a step given for the whole tensor, clipped
constexpr int kRowsFp8 = 3;          // one step per row, FP8 (OCP E4M3) codes: step = absmax / 448
constexpr int kRowsFp8GivenStep = 4; // FP8 codes with a step given for the whole tensor, saturated to +-448
constexpr int kRowsStats = 5;        // as kRowsPerRow, and each row's (mean, rstd) written out (norms only)

// One row of a per-tensor pass: MODE kRowsAmax writes the row's max |y| alone
// (the first pass of a per-tensor dynamic step); kRowsGivenStep writes the
// codes of y with a step given for the whole tensor (the second pass, or a
// static calibrated step), clipped to [-127, 127] (with the FP8 quantiser:
// E4M3 codes saturated to +-448), and x_scale[row] = step if write_scale.
// Either way NONE needs a single pass over the row: each vector's
// raw buffer is refilled with the next row as soon as it has been read.
template <int MODE, typename T, int NORM, int NV, int THREADS, int GREG, int GLDS, typename Q>
__device__ __forceinline__ void quantize_row_tensor(RawRow<T, NV, THREADS>& raw, const void* __restrict__ x,
                                                    int64_t row, int64_t next, int M, int K,
                                                    const float* __restrict__ gamma,
                                                    const ColVec<NV, THREADS, GREG, GLDS>& gv,
                                                    const float* __restrict__ beta, float eps,
                                                    int8_t* __restrict__ xq, float* __restrict__ x_scale,
                                                    RedRing<THREADS>& red, int& rk, const Q& qz,
                                                    bool write_scale) {
  const int nvec = K >> 3;
  using RR = RawRow<T, NV, THREADS>;
  const __amdgpu_buffer_rsrc_t rq = buf_rsrc(xq + row * K, static_cast<uint32_t>(K));
  const bool refill = next < M;
  const __amdgpu_buffer_rsrc_t rn = RR::rsrc(x, next, K);          // used only when refill holds
  constexpr bool amax_only = MODE == kRowsAmax;
  float amax = 0.0f;
  if constexpr (NORM == SQ_NORM_NONE) {
    // Where each vector is refilled right after it is read, wait for the whole
    // row once first: otherwise the compiler, unable to tell the vectors'
    // pending loads apart across the per-vector branches, drains every
    // outstanding load (this row's refills included) before each vector.
    constexpr bool kKeepY = THREADS <= 512 && Storage<T>::kBytes == 2 && NV <= 5;
    if constexpr (amax_only || !kKeepY) __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    if constexpr (amax_only) {
      // one running max, and each vector's raw buffer refilled as soon as it is read
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int vi = threadIdx.x + i * THREADS;
        if (vi < nvec) {
          float y[8];
          none_y(raw, i, gv, y);
#pragma unroll
          for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(y[e]));
          if (refill) raw_load_buf<T>(rn, RR::off(i), raw.r[i]);
        }
      }
    } else if constexpr (kKeepY) {
      // short rows: y of the whole row in registers, the next row requested
      // at once, then the codes (the next row's loads overlap the stores)
      float ys[NV][8];
#pragma unroll
      for (int i = 0; i < NV; ++i)
        if (static_cast<int>(threadIdx.x) + i * THREADS < nvec) none_y(raw, i, gv, ys[i]);
      if (refill) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          const int vi = threadIdx.x + i * THREADS;
          if (vi < nvec) raw_load_buf<T>(rn, RR::off(i), raw.r[i]);
        }
      }
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int vi = threadIdx.x + i * THREADS;
        if (vi < nvec) store_codes8_buf(rq, static_cast<uint32_t>(vi) * 8, qz.template codes8<true>(ys[i]));
      }
    } else {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int vi = threadIdx.x + i * THREADS;
        if (vi < nvec) {
          float y[8];
          none_y(raw, i, gv, y);
          store_codes8_buf(rq, static_cast<uint32_t>(vi) * 8, qz.template codes8<true>(y));
          if (refill) raw_load_buf<T>(rn, RR::off(i), raw.r[i]);
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
        if (vi < nvec) raw_load_buf<T>(rn, RR::off(i), raw.r[i]);
      }
    }
    normalize_row<NORM, NV, THREADS>(v, K, gamma, beta, eps, red, rk);
    if constexpr (amax_only) {
#pragma unroll
      for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[i][e]));
    } else {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int vi = threadIdx.x + i * THREADS;
        if (vi < nvec) store_codes8_buf(rq, static_cast<uint32_t>(vi) * 8, qz.template codes8<true>(v[i]));
      }
    }
  }
  if constexpr (amax_only) {
    amax = block_max<THREADS>(amax, reinterpret_cast<float*>(red.at(rk++)));
    if (threadIdx.x == 0) x_scale[row] = amax;
  } else if (write_scale && threadIdx.x == 0) {
    x_scale[row] = qz.step;
  }
}

// Fused norm + per-token quantisation. Workgroup b handles rows b, b + G, ...
// (G = gridDim.x <= M); one raw row buffer, refilled with the next row while
// the current one is being processed.
template <typename T, int NORM, int NV, int THREADS, int MODE = kRowsPerRow>
__global__ __launch_bounds__(THREADS) void k_norm_quant(const void* __restrict__ x, int M, int K,
                                                        const float* __restrict__ gamma,
                                                        const float* __restrict__ beta, float eps,
                                                        int8_t* __restrict__ xq, float* __restrict__ x_scale,
                                                        const float* __restrict__ step_ptr, int write_scale,
                                                        float* __restrict__ stats) {
  __shared__ RedRing<THREADS> red;
  // NONE keeps its column factors for the workgroup's lifetime (the norms read
  // gamma / beta once per row)
  constexpr int kReg = NORM == SQ_NORM_NONE ? ColSplit<T, NV, THREADS>::kReg : 0;
  constexpr int kLds = NORM == SQ_NORM_NONE ? ColSplit<T, NV, THREADS>::kLds : 0;
  __shared__ float4 gl[kLds > 0 ? 2 * kLds * THREADS : 1];
  // the norms' per-token passes keep gamma / beta of their first vectors on chip
  constexpr bool kPerToken = !(MODE == kRowsAmax || MODE == kRowsGivenStep || MODE == kRowsFp8GivenStep);
  constexpr int kGB = kPerToken ? norm_cache_vectors<NORM, NV, THREADS>() : 0;
  using NC = NormCache<NORM, kGB, THREADS>;
  __shared__ float4 gbl[NC::kFloat4];
  ColVec<NV, THREADS, kReg, kLds> gv;
  const int64_t G = gridDim.x;
  RawRow<T, NV, THREADS> raw;
  raw.load(x, blockIdx.x, K);
  gv.init(NORM == SQ_NORM_NONE ? gamma : nullptr, K >> 3, gl);
  NC::init(gbl, gamma, beta, K >> 3);
  int rk = 0;
  if constexpr (MODE == kRowsAmax || MODE == kRowsGivenStep || MODE == kRowsFp8GivenStep) {
    // per-tensor passes (step_ptr and write_scale are used only here); the FP8
    // code pass is the INT8 one with E4M3 codes
    using Q = typename std::conditional<MODE == kRowsFp8GivenStep, QuantizerFp8, Quantizer>::type;
    constexpr int kPass = MODE == kRowsFp8GivenStep ? kRowsGivenStep : MODE;
    const Q qz(MODE == kRowsAmax ? 0.0f : *step_ptr);
    for (int64_t row = blockIdx.x; row < M; row += G)
      quantize_row_tensor<kPass, T, NORM, NV, THREADS>(raw, x, row, row + G, M, K, gamma, gv, beta, eps, xq, x_scale,
                                                       red, rk, qz, write_scale != 0);
  } else {
    for (int64_t row = blockIdx.x; row < M; row += G)
      quantize_row<T, NORM, NV, THREADS, kReg, kLds, MODE == kRowsFp8, MODE == kRowsStats, kGB>(
          raw, x, row, row + G, M, K, gamma, gv, beta, eps, xq, x_scale, red, rk, stats, gbl);
  }
}

// ----------------------------------------------------------------------------- row layouts (host)

struct RowCfg { int threads, nv; };

// Smallest (threads, vectors per thread) covering K/8 vectors of the row. The
// NONE quantiser of 16-bit rows of 65544 .. 81920 columns takes 512 threads x
// 20 vectors instead of 1024 x 10: one workgroup per CU then holds all of its
// column factors (13 vectors in registers, 7 in LDS) where the 1024-thread
// layout has room for 7 of 10.
inline RowCfg row_cfg(int K, int norm, int bytes) {
  const int nvec = K >> 3;
  if (norm == SQ_NORM_NONE && bytes == 2 && nvec > 8192 && nvec <= 10240) return {512, 20};
  static const RowCfg table[] = {{256, 1}, {256, 2}, {256, 3}, {256, 4}, {512, 3},  {512, 4},   {512, 5},
                                 {512, 6}, {1024, 4}, {1024, 6}, {1024, 8}, {1024, 10}, {1024, 13}, {1024, 17}};
  for (const RowCfg& c : table)
    if (c.threads * c.nv >= nvec) return c;
  return {1024, 17};
}

// Workgroups that fit on the device at once (all CUs x the kernel's occupancy).
inline hipError_t resident_blocks(const void* kernel, int threads, int* out) {
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0);
  *out = (e == hipSuccess) ? cus * (per_cu > 0 ? per_cu : 1) : 0;
  return e;
}


// Calls f.template run<NV, THREADS>() for the row layout of K (as row_cfg); WIDE
// says whether the 512-thread x 20-vector NONE layout is instantiated.
template <bool WIDE, typename F>
hipError_t with_row_cfg(int K, int norm, int bytes, const F& f) {
  const RowCfg c = row_cfg(K, norm, bytes);
  if constexpr (WIDE) {
    if (c.threads == 512 && c.nv == 20) return f.template run<20, 512>();
  }
#define SQ_ROW_CASE(TH, NVV) \
  if (c.threads == TH && c.nv == NVV) return f.template run<NVV, TH>();
  SQ_ROW_CASE(256, 1) SQ_ROW_CASE(256, 2) SQ_ROW_CASE(256, 3) SQ_ROW_CASE(256, 4)
  SQ_ROW_CASE(512, 3) SQ_ROW_CASE(512, 4) SQ_ROW_CASE(512, 5) SQ_ROW_CASE(512, 6)
  SQ_ROW_CASE(1024, 4) SQ_ROW_CASE(1024, 6) SQ_ROW_CASE(1024, 8) SQ_ROW_CASE(1024, 10)
  SQ_ROW_CASE(1024, 13) SQ_ROW_CASE(1024, 17)
#undef SQ_ROW_CASE
  return hipErrorInvalidValue;
}

// Fused norm + quantisation launch: one workgroup per row up to what fits on the device at once.
template <typename T, int NORM, int NV, int THREADS, int MODE>
hipError_t launch_nq(const RowArgs& a, const float* step_ptr, int write_scale, hipStream_t st) {
  auto kern = k_norm_quant<T, NORM, NV, THREADS, MODE>;
  int cap = 0;
  if (hipError_t e = resident_blocks(reinterpret_cast<const void*>(kern), THREADS, &cap)) return e;
  const int grid = static_cast<int>(a.rows < cap ? a.rows : cap);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(THREADS), 0, st, a.x, static_cast<int>(a.rows), a.K, a.gamma, a.beta,
                     a.eps, a.xq, a.x_scale, step_ptr, write_scale, a.stats);
  return hipGetLastError();
}


// Launch the MODE pass of the fused kernel for a's dtype, norm and row layout.
template <int MODE>
struct ModeLaunch {
  template <typename T, int NORM>
  struct L {
    const RowArgs& a;
    const float* step;
    int write_scale;
    hipStream_t st;
    template <int NV, int THREADS>
    hipError_t run() const { return launch_nq<T, NORM, NV, THREADS, MODE>(a, step, write_scale, st); }
  };
  template <typename T>
  static hipError_t norm(const RowArgs& a, const float* step, int write_scale, hipStream_t st) {
    constexpr int B = Storage<T>::kBytes;
    switch (a.norm) {
      case SQ_NORM_NONE:
        return with_row_cfg<B == 2>(a.K, SQ_NORM_NONE, B, L<T, SQ_NORM_NONE>{a, step, write_scale, st});
      case SQ_NORM_LAYERNORM:
        return with_row_cfg<false>(a.K, SQ_NORM_LAYERNORM, B, L<T, SQ_NORM_LAYERNORM>{a, step, write_scale, st});
      case SQ_NORM_RMSNORM:
        return with_row_cfg<false>(a.K, SQ_NORM_RMSNORM, B, L<T, SQ_NORM_RMSNORM>{a, step, write_scale, st});
    }
    return hipErrorInvalidValue;
  }
  static hipError_t run(const RowArgs& a, const float* step, int write_scale, hipStream_t st) {
    switch (a.dtype) {
      case SQ_DT_F32: return norm<f32_t>(a, step, write_scale, st);
      case SQ_DT_F16: return norm<f16_t>(a, step, write_scale, st);
      case SQ_DT_BF16: return norm<bf16_t>(a, step, write_scale, st);
      default: return hipErrorInvalidValue;
    }
  }
};

}  // namespace sq
