// INT8 x INT8 -> INT32 GEMM with the dequantising epilogue, for gfx950.
//
//   y[m, n] = cvt(fl32(fl32(fl32(acc) * x_scale[m]) * w_scale[n]) (+ bias[n])),
//   acc[m, n] = sum_k xq[m, k] * wq[n, k]   (both operands K-contiguous)
//
// Two kernels:
//  * k_gemm_tile  -- prefill shapes. 256x256 output tile per workgroup of eight
//    waves (2 x 4, 128 x 64 each: two waves per SIMD, accumulators in VGPRs), K staged through LDS in 128-byte slices with
//    buffer->LDS DMA (buffer_load_dwordx4 ... lds) into a double buffer, computed
//    with v_mfma_i32_16x16x64_i8. The LDS rows are XOR-swizzled in 16-byte
//    chunks so the fragment reads are bank-conflict free. Workgroups are mapped
//    to tiles XCD by XCD and in column groups, so tiles that share operand rows
//    run at the same time on the same L2.
//  * k_gemm_skinny -- decode shapes (M <= 64), bound by streaming wq from HBM.
//    A workgroup owns 16 output channels; its four waves split K, each streams
//    its 16 rows of wq straight into MFMA operands and the partial accumulators
//    are summed through LDS.
//
// MFMA operand order: the A operand (rows = lane % 16) carries 16 rows of wq and
// the B operand (columns = lane % 16) 16 rows of xq, so the 16x16 result tile
// is acc^T: lane l holds acc[m = l % 16][n = 4 * (l / 16) + r], r = 0..3, four
// consecutive outputs of one token -- one vector store each. Inside one MFMA,
// lane group l / 16 supplies 16 bytes of K for both operands; any assignment of
// K bytes to groups gives the same sum as long as both operands use it.
#include "sq_device.h"
#include "sq_launch.h"
#include "smoothquant.h"

namespace sq {

typedef int v4i __attribute__((ext_vector_type(4)));

// ----------------------------------------------------------------------------- epilogue

// Four consecutive outputs y[m, n .. n+3] of one lane (n % 4 == 0).
template <int YDT>
__device__ __forceinline__ void store4(void* __restrict__ y, int N, int m, int n, const v4i acc, float xs,
                                       const float* __restrict__ ws, const float* __restrict__ bias) {
  const int64_t off = static_cast<int64_t>(m) * N + n;
  const bool full = (n + 3 < N) && ((N & 3) == 0);
  if constexpr (YDT == SQ_DT_I32) {
    int* p = static_cast<int*>(y) + off;
    if (full) {
      *reinterpret_cast<int4*>(p) = make_int4(acc[0], acc[1], acc[2], acc[3]);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (n + r < N) p[r] = acc[r];
    }
    return;
  } else {
    float o[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int nn = min(n + r, N - 1);
      float t = mul_rn(mul_rn(static_cast<float>(acc[r]), xs), ws[nn]);
      if (bias) t = add_rn(t, bias[nn]);
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
      for (int r = 0; r < 4; ++r) h[r] = (YDT == SQ_DT_F16) ? f32_to_f16_rne(o[r]) : f32_to_bf16_rne(o[r]);
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

// ----------------------------------------------------------------------------- tiled kernel

constexpr int kTile = 256;        // output tile edge (m and n)
constexpr int kSlice = 128;       // K bytes per LDS stage
constexpr int kStageBytes = kTile * kSlice;   // one operand, one stage: 32 KiB

// 16-byte chunk position of chunk c in LDS row r (bank-conflict-free fragment
// reads for both 8- and 16-lane access phases).
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Workgroup -> tile. Consecutive workgroup ids land on different XCDs (round
// robin over 8), so ids are first regrouped so that each XCD receives a
// contiguous range of tile numbers; tile numbers then walk `group` tile-rows
// at a time, so concurrently running tiles share rows of xq and wq.
__device__ __forceinline__ void map_tile(int bid, int nwg, int tiles_m, int group, int& tm, int& tn) {
  const int q = nwg >> 3, rem = nwg & 7;
  const int xcd = bid & 7, idx = bid >> 3;
  const int t = (xcd < rem ? xcd * (q + 1) : rem * (q + 1) + (xcd - rem) * q) + idx;
  const int per_group = group * (nwg / tiles_m);         // tiles in one band of `group` tile-rows
  const int g = t / per_group;
  const int first = g * group;
  const int gsz = min(tiles_m - first, group);
  const int within = t - g * per_group;
  tm = first + within % gsz;
  tn = within / gsz;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Raw buffer resource over `base` (uniform); offsets are 32-bit byte offsets.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), 0x7fffffff, 0x00020000);
}

// One operand's slice (256 rows x 128 bytes) into LDS: 4 DMA instructions per
// wave, each filling 8 LDS rows (1 KiB). HALF: only K chunks 0..3 exist (the
// 64-byte tail of K), the other lanes stay idle.
template <bool HALF>
__device__ __forceinline__ void issue_slice(__amdgpu_buffer_rsrc_t rsrc, int8_t* lds, const uint32_t (&off)[4],
                                            int k0, int wid, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (HALF && ((lane & 7) ^ swz((wid * 4 + i) * 8 + (lane >> 3))) >= 4) continue;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(lds + (wid * 4 + i) * 1024), 16, off[i], k0, 0, 0);
  }
}

// Per wave: TI x TJ tiles of 16 x 16 (128 tokens x 64 channels).
constexpr int TI = 8, TJ = 4;

// NSUB 64-byte K steps out of one LDS slice into the accumulator tiles.
template <int NSUB>
__device__ __forceinline__ void mma_slice(const int8_t* la, const int8_t* lb, const int (&a_rd)[2],
                                          const int (&b_rd)[2], v4i (&acc)[TI][TJ]) {
#pragma unroll
  for (int ks = 0; ks < NSUB; ++ks) {
    v4i a[TI], b[TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i) a[i] = *reinterpret_cast<const v4i*>(la + a_rd[ks] + i * 16 * kSlice);
#pragma unroll
    for (int j = 0; j < TJ; ++j) b[j] = *reinterpret_cast<const v4i*>(lb + b_rd[ks] + j * 16 * kSlice);
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(b[j], a[i], acc[i][j], 0, 0, 0);
  }
}

template <int YDT, bool TAIL>
__global__ __launch_bounds__(512, 1) void k_gemm_tile(const int8_t* __restrict__ xq, const float* __restrict__ xs,
                                                      const int8_t* __restrict__ wq, const float* __restrict__ ws,
                                                      const float* __restrict__ bias, void* __restrict__ y,
                                                      int M, int N, int K, int tiles_m, int tiles_n, int group) {
  // Two stages of both operands. Separate arrays let the compiler see that the
  // DMA into one stage never aliases the fragment reads of the other, so it
  // does not wait for the DMA before reading.
  __shared__ __attribute__((aligned(1024))) int8_t lA0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) int8_t lB0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) int8_t lA1[kStageBytes];
  __shared__ __attribute__((aligned(1024))) int8_t lB1[kStageBytes];

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: LDS bases stay scalar
  int tm, tn;
  map_tile(blockIdx.x, tiles_m * tiles_n, tiles_m, group, tm, tn);
  const int m0 = tm * kTile, n0 = tn * kTile;

  // DMA lanes: instruction i of wave w fills LDS rows (w*4 + i)*8 .. +8 of one
  // operand; lane -> row (lane / 8), 16-byte slot (lane % 8), which holds K
  // chunk slot ^ swz(row). Rows past M or N re-read the last row (never stored).
  uint32_t a_off[4], b_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (wid * 4 + i) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz(r);
    a_off[i] = static_cast<uint32_t>(min(m0 + r, M - 1) - m0) * static_cast<uint32_t>(K) + 16u * c;
    b_off[i] = static_cast<uint32_t>(min(n0 + r, N - 1) - n0) * static_cast<uint32_t>(K) + 16u * c;
  }
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(xq + static_cast<int64_t>(m0) * K);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(wq + static_cast<int64_t>(n0) * K);

  // Fragment reads: row R = base + 16 i + lane % 16, K chunk 4 ks + lane / 16.
  const int wm = (wid & 1) * 128, wn = (wid >> 1) * 64;
  int a_rd[2], b_rd[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int rra = wm + (lane & 15), rrb = wn + (lane & 15);
    const int c = 4 * ks + (lane >> 4);
    a_rd[ks] = rra * kSlice + 16 * (c ^ swz(rra));
    b_rd[ks] = rrb * kSlice + 16 * (c ^ swz(rrb));
  }

  v4i acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  // Full 128-byte slices ping-pong between the two stages. The loop body is one
  // straight-line block (the accumulators then stay in AGPRs): each half waits
  // for its stage, issues the next slice into the other stage -- clamped to the
  // last slice, so the final issue is a harmless reload nobody reads -- and
  // multiplies. An odd slice count leaves one slice in stage 0; TAIL adds the
  // 64-byte remainder of K.
  const int nk = K / kSlice;
  const int last = nk > 0 ? (nk - 1) * kSlice : 0;
  if (nk > 0) {
    issue_slice<false>(ra, lA0, a_off, 0, wid, lane);
    issue_slice<false>(rb, lB0, b_off, 0, wid, lane);
  }
  for (int kt = 0; kt + 1 < nk; kt += 2) {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's DMA into stage 0 landed
    __syncthreads();                      // ... every wave's; stage 1 is free again
    issue_slice<false>(ra, lA1, a_off, (kt + 1) * kSlice, wid, lane);
    issue_slice<false>(rb, lB1, b_off, (kt + 1) * kSlice, wid, lane);
    mma_slice<2>(lA0, lB0, a_rd, b_rd, acc);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    const int k2 = min((kt + 2) * kSlice, last);
    issue_slice<false>(ra, lA0, a_off, k2, wid, lane);
    issue_slice<false>(rb, lB0, b_off, k2, wid, lane);
    mma_slice<2>(lA1, lB1, a_rd, b_rd, acc);
  }
  if (nk & 1) {
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    mma_slice<2>(lA0, lB0, a_rd, b_rd, acc);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);     // no DMA outstanding past this point
  if constexpr (TAIL) {
    __syncthreads();
    issue_slice<true>(ra, lA1, a_off, nk * kSlice, wid, lane);
    issue_slice<true>(rb, lB1, b_off, nk * kSlice, wid, lane);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    mma_slice<1>(lA1, lB1, a_rd, b_rd, acc);
  }

  // Epilogue: lane holds acc[m = .. + lane % 16][n = .. + 4 (lane / 16) + r].
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    const int m = m0 + wm + 16 * i + (lane & 15);
    if (m >= M) continue;
    const float xsm = (YDT == SQ_DT_I32) ? 0.0f : xs[m];
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int n = n0 + wn + 16 * j + 4 * (lane >> 4);
      if (n < N) store4<YDT>(y, N, m, n, acc[i][j], xsm, ws, bias);
    }
  }
}

// ----------------------------------------------------------------------------- skinny kernel

template <int MT, int YDT>
__global__ __launch_bounds__(256) void k_gemm_skinny(const int8_t* __restrict__ xq, const float* __restrict__ xs,
                                                     const int8_t* __restrict__ wq, const float* __restrict__ ws,
                                                     const float* __restrict__ bias, void* __restrict__ y,
                                                     int M, int N, int K) {
  __shared__ v4i red[4][MT][64];
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int n0 = blockIdx.x * 16;
  const int kb = 16 * (lane >> 4);
  const int8_t* wrow = wq + static_cast<int64_t>(min(n0 + (lane & 15), N - 1)) * K + kb;
  const int8_t* xrow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) xrow[t] = xq + static_cast<int64_t>(min(16 * t + (lane & 15), M - 1)) * K + kb;

  const int steps = K >> 6;                       // 64-byte K steps
  const int s0 = (steps * wid) >> 2, s1 = (steps * (wid + 1)) >> 2;
  v4i acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = v4i{0, 0, 0, 0};

  constexpr int U = 8;
  int s = s0;
  for (; s + U <= s1; s += U) {
    v4i a[U], b[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u) a[u] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wrow + (s + u) * 64));
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < MT; ++t) b[u][t] = *reinterpret_cast<const v4i*>(xrow[t] + (s + u) * 64);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[u], b[u][t], acc[t], 0, 0, 0);
  }
  for (; s < s1; ++s) {
    const v4i a = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wrow + s * 64));
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const v4i b = *reinterpret_cast<const v4i*>(xrow[t] + s * 64);
      acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[t], 0, 0, 0);
    }
  }
#pragma unroll
  for (int t = 0; t < MT; ++t) red[wid][t][lane] = acc[t];
  __syncthreads();
  // wave w finishes m-tiles t = w, w + 4, ...
  for (int t = wid; t < MT; t += 4) {
    const v4i tot = red[0][t][lane] + red[1][t][lane] + red[2][t][lane] + red[3][t][lane];
    const int m = 16 * t + (lane & 15);
    const int n = n0 + 4 * (lane >> 4);
    if (m < M && n < N) store4<YDT>(y, N, m, n, tot, (YDT == SQ_DT_I32) ? 0.0f : xs[m], ws, bias);
  }
}

// ----------------------------------------------------------------------------- dispatch

namespace {

template <int YDT>
hipError_t launch_typed(const GemmArgs& g, hipStream_t st) {
  if (g.M <= 64) {
    const dim3 grid((g.N + 15) / 16);
    const int mt = (g.M + 15) / 16;
#define SQ_SKINNY(MTV)                                                                                       \
  case MTV:                                                                                                  \
    hipLaunchKernelGGL((k_gemm_skinny<MTV, YDT>), grid, dim3(256), 0, st, g.xq, g.x_scale, g.wq, g.w_scale, \
                       g.bias, g.y, g.M, g.N, g.K);                                                          \
    break;
    switch (mt) {
      SQ_SKINNY(1) SQ_SKINNY(2) SQ_SKINNY(3) SQ_SKINNY(4)
      default: return hipErrorInvalidValue;
    }
#undef SQ_SKINNY
    return hipGetLastError();
  }
  const int tiles_m = (g.M + kTile - 1) / kTile;
  const int tiles_n = (g.N + kTile - 1) / kTile;
  const int group = min(tiles_m, 8);
  if (g.K % kSlice)
    hipLaunchKernelGGL((k_gemm_tile<YDT, true>), dim3(tiles_m * tiles_n), dim3(512), 0, st, g.xq, g.x_scale, g.wq,
                       g.w_scale, g.bias, g.y, g.M, g.N, g.K, tiles_m, tiles_n, group);
  else
    hipLaunchKernelGGL((k_gemm_tile<YDT, false>), dim3(tiles_m * tiles_n), dim3(512), 0, st, g.xq, g.x_scale,
                       g.wq, g.w_scale, g.bias, g.y, g.M, g.N, g.K, tiles_m, tiles_n, group);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& g, hipStream_t st) {
  switch (g.y_dt) {
    case SQ_DT_F32: return launch_typed<SQ_DT_F32>(g, st);
    case SQ_DT_F16: return launch_typed<SQ_DT_F16>(g, st);
    case SQ_DT_BF16: return launch_typed<SQ_DT_BF16>(g, st);
    case SQ_DT_I32: return launch_typed<SQ_DT_I32>(g, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace sq
