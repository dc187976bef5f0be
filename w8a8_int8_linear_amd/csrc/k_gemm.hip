// INT8 x INT8 -> INT32 GEMM with the dequantising epilogue, for gfx950.
//
//   y[m, n] = cvt(fl32(fl32(fl32(acc) * x_scale[m]) * w_scale[n]) (+ bias[n])),
//   acc[m, n] = sum_k xq[m, k] * wq[n, k]   (both operands K-contiguous)
//
// Two kernels:
//  * k_gemm_tile  -- prefill shapes. 256x256 output tile per workgroup of eight
//    waves (2 x 4, 128 x 64 each: two waves per SIMD, accumulators in VGPRs), K
//    staged through LDS in 64-byte slices by buffer->LDS DMA
//    (buffer_load_dwordx4 ... lds) into a 4-stage ring with three slices in
//    flight, computed with v_mfma_i32_16x16x64_i8. LDS rows are swizzled in
//    16-byte chunks so the fragment reads are bank-conflict free. Workgroups are
//    mapped to tiles XCD by XCD and in column groups, so tiles that share
//    operand rows run at the same time on the same L2.
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

constexpr int kTile = 256;                     // output tile edge (m and n)
constexpr int kSlice = 64;                     // K bytes per LDS stage: one MFMA K step
constexpr int kStages = 4;                     // LDS ring depth: slices in flight = kStages - 1
constexpr int kStageBytes = kTile * kSlice;    // one operand, one stage: 16 KiB
constexpr int kDmaPerWave = kStageBytes / 1024 / 8;   // 1 KiB DMA instructions per wave per operand: 2

// LDS layout of a stage: row r of the operand at r * 64, its 16-byte K chunk c
// at slot c ^ swz(r). A ds_read_b128 serves 32 lanes at a time from a 512-byte
// window; a fragment read has lanes 0..31 on 16 rows x 2 chunks, and rows r,
// r + 8 share a window position, so they get slots differing in bit 1.
__device__ __forceinline__ int swz(int r) { return ((r >> 3) & 1) << 1; }

// Workgroup -> tile. Consecutive workgroup ids land on different XCDs (round
// robin over 8), so ids are first regrouped so that each XCD receives a
// contiguous range of tile numbers; tile numbers then walk `group` tile-rows
// at a time, so concurrently running tiles share rows of xq and wq in L2.
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

// Workgroup barrier without the release/acquire fences of __syncthreads (those
// would drain every outstanding DMA, vmcnt(0)). The memory clobber keeps the
// compiler from moving LDS accesses across it; visibility of the DMA data
// comes from each wave's own vmcnt wait before the barrier.
__device__ __forceinline__ void stage_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Raw buffer resource over `base` (uniform); offsets are 32-bit byte offsets.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), 0x7fffffff, 0x00020000);
}

// One operand's slice (256 rows x 64 bytes) into LDS: kDmaPerWave DMA
// instructions per wave, each filling 16 LDS rows (1 KiB).
__device__ __forceinline__ void issue_slice(__amdgpu_buffer_rsrc_t rsrc, int8_t* lds, const uint32_t (&off)[kDmaPerWave],
                                            int k0, int wid) {
#pragma unroll
  for (int i = 0; i < kDmaPerWave; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(lds + (wid * kDmaPerWave + i) * 1024), 16, off[i], k0,
                                             0, 0);
}

// Per wave: TI x TJ tiles of 16 x 16 (128 tokens x 64 channels).
constexpr int TI = 8, TJ = 4;

// Fragments of one 64-byte K step: TI tiles of xq rows and TJ tiles of wq rows.
struct Frags {
  v4i a[TI], b[TJ];
};

__device__ __forceinline__ void read_frags(const int8_t* la, const int8_t* lb, int a_rd, int b_rd, Frags& f) {
#pragma unroll
  for (int i = 0; i < TI; ++i) f.a[i] = *reinterpret_cast<const v4i*>(la + a_rd + i * 16 * kSlice);
#pragma unroll
  for (int j = 0; j < TJ; ++j) f.b[j] = *reinterpret_cast<const v4i*>(lb + b_rd + j * 16 * kSlice);
}

// Scheduling of one step: each fragment read of the next slice goes out
// between MFMAs of the current one (the MFMAs only need registers read a step
// earlier), and nothing crosses the end of the step -- the compiler would
// otherwise hoist the next step's MFMAs above the stage barrier, right behind
// the reads they depend on.
__device__ __forceinline__ void interleave_reads_with_mfma() {
#pragma unroll
  for (int i = 0; i < TI + TJ; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // 1 LDS read
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // 2 MFMA
  }
  __builtin_amdgcn_sched_group_barrier(0x008, TI * TJ - 2 * (TI + TJ), 0);
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void mma(const Frags& f, v4i (&acc)[TI][TJ]) {
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
}

template <int YDT>
__global__ __launch_bounds__(512, 1) void k_gemm_tile(const int8_t* __restrict__ xq, const float* __restrict__ xs,
                                                      const int8_t* __restrict__ wq, const float* __restrict__ ws,
                                                      const float* __restrict__ bias, void* __restrict__ y,
                                                      int M, int N, int K, int tiles_m, int tiles_n, int group) {
  // Ring of kStages stages per operand, each its own array: the compiler then
  // sees that a DMA into one stage never aliases the fragment reads of another
  // and inserts no wait of its own before those reads.
  __shared__ __attribute__((aligned(1024))) int8_t lA0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) int8_t lA1[kStageBytes];
  __shared__ __attribute__((aligned(1024))) int8_t lA2[kStageBytes];
  __shared__ __attribute__((aligned(1024))) int8_t lA3[kStageBytes];
  __shared__ __attribute__((aligned(1024))) int8_t lB0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) int8_t lB1[kStageBytes];
  __shared__ __attribute__((aligned(1024))) int8_t lB2[kStageBytes];
  __shared__ __attribute__((aligned(1024))) int8_t lB3[kStageBytes];

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: LDS bases stay scalar
  int tm, tn;
  map_tile(blockIdx.x, tiles_m * tiles_n, tiles_m, group, tm, tn);
  const int m0 = tm * kTile, n0 = tn * kTile;

  // DMA lanes: instruction i of wave w fills LDS rows (w*2 + i)*16 .. +16 of one
  // operand; lane -> row (lane / 4), 16-byte slot (lane % 4), which holds K
  // chunk slot ^ swz(row). Rows past M or N re-read the last row (never stored).
  uint32_t a_off[kDmaPerWave], b_off[kDmaPerWave];
#pragma unroll
  for (int i = 0; i < kDmaPerWave; ++i) {
    const int r = (wid * kDmaPerWave + i) * 16 + (lane >> 2);
    const int c = (lane & 3) ^ swz(r);
    a_off[i] = static_cast<uint32_t>(min(m0 + r, M - 1) - m0) * static_cast<uint32_t>(K) + 16u * c;
    b_off[i] = static_cast<uint32_t>(min(n0 + r, N - 1) - n0) * static_cast<uint32_t>(K) + 16u * c;
  }
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(xq + static_cast<int64_t>(m0) * K);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(wq + static_cast<int64_t>(n0) * K);

  // Fragment reads: row R = base + 16 i + lane % 16, K chunk lane / 16.
  const int wm = (wid & 1) * 128, wn = (wid >> 1) * 64;
  const int rra = wm + (lane & 15), rrb = wn + (lane & 15);
  const int a_rd = rra * kSlice + 16 * ((lane >> 4) ^ swz(rra));
  const int b_rd = rrb * kSlice + 16 * ((lane >> 4) ^ swz(rrb));

  v4i acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  // Slices go round the 4-stage ring. At step k the fragments of slice k are
  // already in registers (read during step k - 1); the step waits for slice
  // k + 1 to land (vmcnt(8): each wave always has three slices, 4 DMA
  // instructions each, in flight, since issue indices are clamped to the last
  // slice and the final issues are harmless reloads), lets the barrier make it
  // visible and free the stage slice k was read from, refills that stage with
  // slice k + 4, reads the fragments of slice k + 1 and multiplies slice k
  // meanwhile, so LDS latency hides behind the MFMAs. lgkmcnt(0) before the
  // barrier: this wave's fragment reads of the stage about to be refilled are
  // done.
  const int nk = K / kSlice;
  const int last = (nk - 1) * kSlice;
  issue_slice(ra, lA0, a_off, 0, wid);
  issue_slice(rb, lB0, b_off, 0, wid);
  issue_slice(ra, lA1, a_off, min(kSlice, last), wid);
  issue_slice(rb, lB1, b_off, min(kSlice, last), wid);
  issue_slice(ra, lA2, a_off, min(2 * kSlice, last), wid);
  issue_slice(rb, lB2, b_off, min(2 * kSlice, last), wid);
  issue_slice(ra, lA3, a_off, min(3 * kSlice, last), wid);
  issue_slice(rb, lB3, b_off, min(3 * kSlice, last), wid);
  Frags f0, f1;
  __builtin_amdgcn_s_waitcnt(0x0F7C);     // vmcnt(12): slice 0 landed
  stage_barrier();
  read_frags(lA0, lB0, a_rd, b_rd, f0);

#define SQ_STEP(FC, FN, LA_NEXT, LB_NEXT, LA_FREE, LB_FREE)                 \
  {                                                                     \
    __builtin_amdgcn_s_waitcnt(0x0078); /* vmcnt(8) lgkmcnt(0) */       \
    stage_barrier();                                                    \
    const int kn = min((kt + 4) * kSlice, last);                        \
    issue_slice(ra, LA_FREE, a_off, kn, wid);                           \
    issue_slice(rb, LB_FREE, b_off, kn, wid);                           \
    __builtin_amdgcn_sched_barrier(0);                                  \
    read_frags(LA_NEXT, LB_NEXT, a_rd, b_rd, FN);                       \
    mma(FC, acc);                                                       \
    interleave_reads_with_mfma();                                       \
    ++kt;                                                               \
  }
  int kt = 0;
  for (; kt + 4 <= nk;) {
    SQ_STEP(f0, f1, lA1, lB1, lA0, lB0)
    SQ_STEP(f1, f0, lA2, lB2, lA1, lB1)
    SQ_STEP(f0, f1, lA3, lB3, lA2, lB2)
    SQ_STEP(f1, f0, lA0, lB0, lA3, lB3)
  }
  if (kt < nk) SQ_STEP(f0, f1, lA1, lB1, lA0, lB0)
  if (kt < nk) SQ_STEP(f1, f0, lA2, lB2, lA1, lB1)
  if (kt < nk) SQ_STEP(f0, f1, lA3, lB3, lA2, lB2)
#undef SQ_STEP
  __builtin_amdgcn_s_waitcnt(0x0070);     // vmcnt(0) lgkmcnt(0): no DMA into LDS outlives the loop

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
  hipLaunchKernelGGL((k_gemm_tile<YDT>), dim3(tiles_m * tiles_n), dim3(512), 0, st, g.xq, g.x_scale, g.wq,
                     g.w_scale, g.bias, g.y, g.M, g.N, g.K, tiles_m, tiles_n, group);
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
