// INT8 x INT8 -> INT32 GEMM with the dequantising epilogue, for gfx950.
//
//   y[m, n] = cvt(fl32(fl32(fl32(acc) * x_scale[m]) * w_scale[n]) (+ bias[n])),
//   acc[m, n] = sum_k xq[m, k] * wq[n, k]   (both operands K-contiguous)
//
// Kernels:
//  * k_gemm_tile  -- prefill shapes. 256x256 output tile per workgroup of eight
//    waves (2 x 4, 128 x 64 each: two waves per SIMD, accumulators in VGPRs), K
//    staged through LDS 128 bytes at a time by buffer->LDS DMA
//    (buffer_load_dwordx4 ... lds) into a 2-stage ring, computed with
//    v_mfma_i32_16x16x64_i8. LDS rows are swizzled in 16-byte chunks so the
//    fragment reads are bank-conflict free. Workgroups are mapped to tiles XCD
//    by XCD and in column groups, so tiles that share operand rows run at the
//    same time on the same L2. Up to 16 tiles per resident workgroup, the
//    grid is one workgroup per CU looping over tiles, the next tile's first
//    stages in flight during each epilogue. k_gemm_tile_k64 is the same tile
//    with 64-byte slices in a 4-stage ring, for K % 128 == 64, one tile per
//    workgroup.
//  * k_gemv (up to 4 tokens at N >= 16384, vector ALUs) and k_gemm_decode
//    (the other shapes up to 128 tokens, MFMA) -- decode shapes, bound by
//    streaming wq from HBM (described at the kernels).
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

#include <type_traits>

namespace sq {

typedef int v4i __attribute__((ext_vector_type(4)));

// ----------------------------------------------------------------------------- epilogue

// Four consecutive outputs y[m, n .. n+3] of one lane (n % 4 == 0).
template <int YDT, typename AccV = v4i>
__device__ __forceinline__ void store4(void* __restrict__ y, int N, int m, int n, const AccV acc, float xs,
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

// store4 with the weight scales of the four outputs already in registers (w
// holds ws[n .. n+3], clamped to the last column): the same roundings, for an
// epilogue that must not wait on memory issued after the scales. The bias, when
// there is one, is read here.
template <int YDT, typename AccV = v4i>
__device__ __forceinline__ void store4_pre(void* __restrict__ y, int N, int m, int n, const AccV acc, float xs,
                                           const float (&w)[4], const float* __restrict__ bias) {
  const int64_t off = static_cast<int64_t>(m) * N + n;
  const bool full = (n + 3 < N) && ((N & 3) == 0);
  if constexpr (YDT == SQ_DT_I32) {
    static_assert(std::is_same_v<AccV, v4i>, "int32 output of an int32 accumulator");
    int* p = static_cast<int*>(y) + off;
    if (full) {
      *reinterpret_cast<int4*>(p) = make_int4(acc[0], acc[1], acc[2], acc[3]);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (n + r < N) p[r] = acc[r];
    }
  } else {
    float o[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float t = mul_rn(mul_rn(static_cast<float>(acc[r]), xs), w[r]);
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

// Outputs of two adjacent 16-column MFMA tiles j, j+1 in a 16-bit type, 16
// bytes per lane. Lane group g = lane / 16 holds columns 4g .. 4g+3 of both
// tiles (rows lane % 16). One v_permlane16_swap per dword exchanges the
// tile-j values of groups 1 and 3 with the tile-(j+1) values of groups 0 and
// 2, after which group g holds 8 consecutive outputs starting at column
// 16 (g & 1) + 8 (g >> 1) of the pair, and one store instruction covers 64
// contiguous bytes of each of its 16 rows (four 32-byte pieces before).
// Measured on the 256x256 tile at K = 4096: the epilogue from 8-13 to 4-6 us
// per tile. Same roundings as store4_pre; w0 / w1 hold the weight scales of
// the lane's columns in tiles j and j+1 (clamped to the last column). Every
// lane takes part in the swaps; the stores are guarded per lane.
template <int YDT, typename AccV = v4i>
__device__ __forceinline__ void store8_pair(void* __restrict__ y, int M, int N, int m, int nb, const AccV a0,
                                            const AccV a1, float xs, const float (&w0)[4], const float (&w1)[4],
                                            const float* __restrict__ bias, int lane) {
  static_assert(YDT == SQ_DT_F16 || YDT == SQ_DT_BF16, "16-bit outputs");
  const int g = lane >> 4;
  uint32_t h[2][4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float t0 = mul_rn(mul_rn(static_cast<float>(a0[r]), xs), w0[r]);
    float t1 = mul_rn(mul_rn(static_cast<float>(a1[r]), xs), w1[r]);
    if (bias) {
      t0 = add_rn(t0, bias[min(nb + 4 * g + r, N - 1)]);
      t1 = add_rn(t1, bias[min(nb + 16 + 4 * g + r, N - 1)]);
    }
    h[0][r] = (YDT == SQ_DT_F16) ? f32_to_f16_rne(t0) : f32_to_bf16_rne(t0);
    h[1][r] = (YDT == SQ_DT_F16) ? f32_to_f16_rne(t1) : f32_to_bf16_rne(t1);
  }
  const auto lo = __builtin_amdgcn_permlane16_swap(h[0][0] | (h[0][1] << 16), h[1][0] | (h[1][1] << 16), false, false);
  const auto hi = __builtin_amdgcn_permlane16_swap(h[0][2] | (h[0][3] << 16), h[1][2] | (h[1][3] << 16), false, false);
  const uint32_t d[4] = {lo[0], hi[0], lo[1], hi[1]};
  const int c = nb + 16 * (g & 1) + 8 * (g >> 1);
  if (m >= M) return;
  uint16_t* p = static_cast<uint16_t*>(y) + static_cast<int64_t>(m) * N + c;
  if (c + 7 < N && (N & 7) == 0) {
    *reinterpret_cast<uint4*>(p) = make_uint4(d[0], d[1], d[2], d[3]);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (c + e < N) p[e] = static_cast<uint16_t>(d[e >> 1] >> (16 * (e & 1)));
  }
}

// ----------------------------------------------------------------------------- tiled kernel

constexpr int kTile = 256;                     // output tile edge (m and n)
constexpr int kSlice = 64;                     // K bytes per LDS stage: one MFMA K step
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
// the reads they depend on. The step's DMA instructions are spread over the
// first MFMAs as well: issued together right after the barrier, the eight
// waves' DMAs queue at the CU's address unit and stall the waves behind them.
__device__ __forceinline__ void interleave_reads_with_mfma() {
  static_assert(2 * kDmaPerWave <= (TI + TJ + 2) / 3, "one DMA per three fragment reads");
#pragma unroll
  for (int i = 0; i < TI + TJ; ++i) {
    if (i % 3 == 0 && i / 3 < 2 * kDmaPerWave) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // 1 DMA
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
__global__ __launch_bounds__(512, 1) void k_gemm_tile_k64(const int8_t* __restrict__ xq, const float* __restrict__ xs,
                                                      const int8_t* __restrict__ wq, const float* __restrict__ ws,
                                                      const float* __restrict__ bias, void* __restrict__ y,
                                                      int M, int N, int K, int tiles_m, int tiles_n, int group) {
  // Ring of four stages per operand, each its own array: the compiler then
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
  // in slice order: the waits below count DMAs in issue order, and the stages
  // being distinct objects the compiler could otherwise interleave them
  issue_slice(ra, lA0, a_off, 0, wid);
  issue_slice(rb, lB0, b_off, 0, wid);
  memory_opaque();
  issue_slice(ra, lA1, a_off, min(kSlice, last), wid);
  issue_slice(rb, lB1, b_off, min(kSlice, last), wid);
  memory_opaque();
  issue_slice(ra, lA2, a_off, min(2 * kSlice, last), wid);
  issue_slice(rb, lB2, b_off, min(2 * kSlice, last), wid);
  memory_opaque();
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
    __builtin_amdgcn_sched_barrier(0);                                  \
    issue_slice(ra, LA_FREE, a_off, kn, wid);                           \
    issue_slice(rb, LB_FREE, b_off, kn, wid);                           \
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
  if constexpr (YDT == SQ_DT_F16 || YDT == SQ_DT_BF16) {
    float wv[TJ][4];
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) wv[j][r] = ws[min(n0 + wn + 16 * j + 4 * (lane >> 4) + r, N - 1)];
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int m = m0 + wm + 16 * i + (lane & 15);
      const float xsm = xs[min(m, M - 1)];
#pragma unroll
      for (int j = 0; j < TJ; j += 2)
        store8_pair<YDT>(y, M, N, m, n0 + wn + 16 * j, acc[i][j], acc[i][j + 1], xsm, wv[j], wv[j + 1], bias, lane);
    }
  } else {
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
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const int8_t* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)(p)));
}

// Fragment reads written in asm: at the top of the ring loop the compiler no
// longer knows which stage each outstanding DMA writes and would drain them
// all (vmcnt(0)) before a plain LDS read. The DMA data is already covered by
// the explicit vmcnt wait ahead of the stage barrier; each asm statement waits
// for its own reads before its outputs are used.
template <int N>
__device__ __forceinline__ void lds_read_frags(v4i (&r)[N], const uint32_t (&a)[N]) {
  int i = 0;
#pragma unroll
  for (; i + 4 <= N; i += 4)
    asm volatile(
        "ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b128 %2, %6\n\tds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[i]), "=&v"(r[i + 1]), "=&v"(r[i + 2]), "=&v"(r[i + 3])
        : "v"(a[i]), "v"(a[i + 1]), "v"(a[i + 2]), "v"(a[i + 3])
        : "memory");
#pragma unroll
  for (; i + 2 <= N; i += 2)
    asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(r[i]), "=&v"(r[i + 1])
                 : "v"(a[i]), "v"(a[i + 1])
                 : "memory");
#pragma unroll
  for (; i < N; ++i)
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(r[i]) : "v"(a[i]) : "memory");
}

// ----------------------------------------------------------------------------- tiled kernel, 128-byte stages

// The same tile and wave layout, with K staged 128 bytes (two MFMA K steps) at
// a time in a 2-stage ring: each DMA instruction then fetches 8 rows x 128
// bytes, whole L2 lines, where a 64-byte stage can only fetch half lines
// (16 rows x 64 bytes). Measured on the MT-NLG shapes: 2810 against 2550
// TOPS. The barrier is needed once per stage, i.e. every second K step.
// Requires K % 128 == 0 (the 64-byte kernel takes the other case).
constexpr int kSlice2 = 128;                         // K bytes per stage
constexpr int kStage2Bytes = kTile * kSlice2;        // one operand, one stage: 32 KiB
constexpr int kDma2PerWave = kStage2Bytes / 1024 / 8;   // DMA instructions (8 rows x 128 B) per wave per operand: 4

// LDS layout of a stage: row r at r * 128, its 16-byte chunk c at slot
// c ^ swz2(r). Lanes 0..31 of a fragment read cover 16 rows x chunks 4t, 4t+1;
// rows r, r + 4, r + 8, r + 12 share a 512-byte window position, so they get
// slot offsets 0, 2, 4, 6 and the 32 lanes hit 32 distinct slots.
__device__ __forceinline__ int swz2(int r) { return ((r >> 2) & 3) << 1; }

// As interleave_reads_with_mfma; on the step that refills a stage, its eight
// DMA instructions go out two at a time between the first MFMAs.
__device__ __forceinline__ void interleave2(bool with_dma) {
  static_assert(2 * kDma2PerWave <= 2 * ((TI + TJ + 2) / 3), "two DMAs per three fragment reads");
#pragma unroll
  for (int i = 0; i < TI + TJ; ++i) {
    if (with_dma && i % 3 == 0 && i / 3 < kDma2PerWave) __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // 1 LDS read
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // 2 MFMA
  }
  __builtin_amdgcn_sched_group_barrier(0x008, TI * TJ - 2 * (TI + TJ), 0);
  __builtin_amdgcn_sched_barrier(0);
}

// The tile's width in N as MFMA tiles per wave, TJN: 4 (256 columns), 3 (192)
// or 2 (128). The eight waves stay 2 x 4, each 128 tokens x 16 TJN channels,
// and a stage's wq rows take TJN DMA instructions per wave. Narrower tiles
// serve short grids: a width whose tile count fills whole waves of the CUs
// wastes less of the last wave (OPT-6.7B's QKV, 2048 x 12288: 384 tiles of
// 256 x 256 are 1.5 waves on 256 CUs, 512 tiles of 256 x 192 are two).
template <int TJN>
struct FragsN {
  v4i a[TI], b[TJN];
};

// Stage rows of one operand: N DMA instructions per wave (8 rows x 128 bytes each).
template <int N>
__device__ __forceinline__ void issue_rows2(__amdgpu_buffer_rsrc_t rsrc, int8_t* lds, const uint32_t* off, int k0,
                                            int wid) {
#pragma unroll
  for (int i = 0; i < N; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(lds + (wid * N + i) * 1024), 16, off[i], k0, 0, 0);
}

template <int TJN>
__device__ __forceinline__ void read_frags2n(const int8_t* la, const int8_t* lb, const int (&a_rd)[2],
                                             const int (&b_rd)[2], int t, FragsN<TJN>& f) {
#pragma unroll
  for (int i = 0; i < TI; ++i) f.a[i] = *reinterpret_cast<const v4i*>(la + a_rd[t] + i * 16 * kSlice2);
#pragma unroll
  for (int j = 0; j < TJN; ++j) f.b[j] = *reinterpret_cast<const v4i*>(lb + b_rd[t] + j * 16 * kSlice2);
}

template <int TJN>
__device__ __forceinline__ void mma_n(const FragsN<TJN>& f, v4i (&acc)[TI][TJN]) {
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
}

// interleave2 for any width: the step's MFMAs spread evenly over its fragment
// reads (1-3 after each), the refill's DMAs two at a time after every third
// read. TJN = 4 keeps interleave2's schedule.
template <int TJN>
__device__ __forceinline__ void interleave2n(bool with_dma) {
  if constexpr (TJN == 4) {
    interleave2(with_dma);
  } else {
    constexpr int NR = TI + TJN, NM = TI * TJN, ND = kDma2PerWave + TJN;
    static_assert(NM >= NR && NM <= 3 * NR && (ND + 1) / 2 <= (NR + 2) / 3, "schedule shape");
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      if (with_dma && i % 3 == 0 && i / 3 < (ND + 1) / 2) __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      const int c = (i + 1) * NM / NR - i * NM / NR;
      if (c == 1) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      else if (c == 2) __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      else __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int YDT, int TJN = 4>
__global__ __launch_bounds__(512, 1) void k_gemm_tile(const int8_t* __restrict__ xq, const float* __restrict__ xs,
                                                      const int8_t* __restrict__ wq, const float* __restrict__ ws,
                                                      const float* __restrict__ bias, void* __restrict__ y, int M,
                                                      int N, int K, int tiles_m, int tiles_n, int group) {
  __shared__ __attribute__((aligned(1024))) int8_t lA0[kStage2Bytes];
  __shared__ __attribute__((aligned(1024))) int8_t lA1[kStage2Bytes];
  __shared__ __attribute__((aligned(1024))) int8_t lB0[kStage2Bytes];   // 64 TJN of its 256 rows used
  __shared__ __attribute__((aligned(1024))) int8_t lB1[kStage2Bytes];
  constexpr int kTN = 64 * TJN;                      // tile width in N

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: LDS bases stay scalar
  const int ntiles = tiles_m * tiles_n;

  // Workgroup b takes tiles b, b + G, b + 2G, ... (G = gridDim.x: ntiles, or
  // a multiple of 8 below it, so each id keeps the XCD that map_tile assumes
  // and the tiles run in the order a one-tile-per-workgroup launch would
  // dispatch them). Per tile: DMA lanes, instruction i of wave w
  // filling LDS rows (w*4 + i)*8 .. +8 of one operand; lane -> row lane / 8,
  // slot lane % 8, which holds chunk slot ^ swz2(row). Rows past M or N
  // re-read the last row (never stored).
  int m0 = 0, n0 = 0;
  uint32_t a_off[kDma2PerWave], b_off[TJN];
  __amdgpu_buffer_rsrc_t ra, rb;
  auto setup = [&](int v) {
    int tm, tn;
    map_tile(v, ntiles, tiles_m, group, tm, tn);
    m0 = tm * kTile;
    n0 = tn * kTN;
    // recomputed per tile from the lane id read afresh (mbcnt in volatile asm
    // cannot be hoisted): kept across the tile loop, these per-lane offsets
    // would hold registers the loop needs
    int ln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
#pragma unroll
    for (int i = 0; i < kDma2PerWave; ++i) {
      const int r = (wid * kDma2PerWave + i) * 8 + (ln >> 3);
      const int c = (ln & 7) ^ swz2(r);
      a_off[i] = static_cast<uint32_t>(min(m0 + r, M - 1) - m0) * static_cast<uint32_t>(K) + 16u * c;
    }
#pragma unroll
    for (int i = 0; i < TJN; ++i) {
      const int r = (wid * TJN + i) * 8 + (ln >> 3);
      const int c = (ln & 7) ^ swz2(r);
      b_off[i] = static_cast<uint32_t>(min(n0 + r, N - 1) - n0) * static_cast<uint32_t>(K) + 16u * c;
    }
    ra = make_rsrc(xq + static_cast<int64_t>(m0) * K);
    rb = make_rsrc(wq + static_cast<int64_t>(n0) * K);
  };

  // Fragment reads of K step t: row R = base + 16 i + lane % 16, chunk 4 t + lane / 16.
  const int wm = (wid & 1) * 128, wn = (wid >> 1) * (16 * TJN);
  const int rra = wm + (lane & 15), rrb = wn + (lane & 15);
  int a_rd[2], b_rd[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int c = 4 * t + (lane >> 4);
    a_rd[t] = rra * kSlice2 + 16 * (c ^ swz2(rra));
    b_rd[t] = rrb * kSlice2 + 16 * (c ^ swz2(rrb));
  }

  // Stage S holds K steps 2S and 2S+1. Entering stage S, the fragments of step
  // 2S are in registers and stage S+1 is in flight. Step 2S reads the
  // fragments of step 2S+1 from the same stage and multiplies step 2S. Step
  // 2S+1 waits for stage S+1 (vmcnt(0): it is the only stage in flight),
  // lets the barrier make it visible and free stage S's buffer (lgkmcnt(0):
  // this wave's reads of it are done), refills that buffer with stage S+2,
  // reads the fragments of step 2S+2 and multiplies step 2S+1. Issue indices
  // are clamped to the last stage; the final issues are harmless reloads.
  const int ns = K / kSlice2;
  const int last = (ns - 1) * kSlice2;
  auto prologue = [&]() {
    // in stage order: the waits count DMAs in issue order (see the 64-byte kernel)
    issue_rows2<kDma2PerWave>(ra, lA0, a_off, 0, wid);
    issue_rows2<TJN>(rb, lB0, b_off, 0, wid);
    memory_opaque();
    issue_rows2<kDma2PerWave>(ra, lA1, a_off, min(kSlice2, last), wid);
    issue_rows2<TJN>(rb, lB1, b_off, min(kSlice2, last), wid);
  };
  int v = blockIdx.x;
  setup(v);
  prologue();

  for (;;) {
    v4i acc[TI][TJN];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJN; ++j) acc[i][j] = v4i{0, 0, 0, 0};
    FragsN<TJN> f0, f1;
    // vmcnt(kStageDma): stage 0 landed. Loads complete in issue order, so with
    // at most as many operations outstanding as stage 1 issued (4 + TJN DMA
    // instructions per wave) no load of stage 0 can be (the previous tile's
    // stores, issued after these DMAs, are waited for as well).
    constexpr int kStageDma = kDma2PerWave + TJN;
    __builtin_amdgcn_s_waitcnt((kStageDma & 15) | ((kStageDma >> 4) << 14) | 0x0F70);
    stage_barrier();
    {
      // in asm: across the tile loop's back edge the compiler's own waits would
      // also drain stage 1 and the previous tile's stores (vmcnt(0))
      uint32_t addr[TI + TJN];
      v4i r[TI + TJN];
#pragma unroll
      for (int i = 0; i < TI; ++i) addr[i] = lds_addr(lA0) + a_rd[0] + i * 16 * kSlice2;
#pragma unroll
      for (int j = 0; j < TJN; ++j) addr[TI + j] = lds_addr(lB0) + b_rd[0] + j * 16 * kSlice2;
      lds_read_frags(r, addr);
#pragma unroll
      for (int i = 0; i < TI; ++i) f0.a[i] = r[i];
#pragma unroll
      for (int j = 0; j < TJN; ++j) f0.b[j] = r[TI + j];
    }

#define SQ_STAGE(LA_CUR, LB_CUR, LA_NXT, LB_NXT)                                      \
  {                                                                                   \
    read_frags2n(LA_CUR, LB_CUR, a_rd, b_rd, 1, f1);                                  \
    mma_n(f0, acc);                                                                   \
    interleave2n<TJN>(false);                                                         \
    __builtin_amdgcn_s_waitcnt(0x0070); /* vmcnt(0) lgkmcnt(0) */                     \
    stage_barrier();                                                                  \
    const int kn = min((s + 2) * kSlice2, last);                                      \
    __builtin_amdgcn_sched_barrier(0);                                                \
    issue_rows2<kDma2PerWave>(ra, LA_CUR, a_off, kn, wid);                                          \
    issue_rows2<TJN>(rb, LB_CUR, b_off, kn, wid);                                          \
    read_frags2n(LA_NXT, LB_NXT, a_rd, b_rd, 0, f0);                                  \
    mma_n(f1, acc);                                                                   \
    interleave2n<TJN>(true);                                                          \
    ++s;                                                                              \
  }
    int s = 0;
    for (; s + 2 <= ns;) {
      SQ_STAGE(lA0, lB0, lA1, lB1)
      SQ_STAGE(lA1, lB1, lA0, lB0)
    }
    if (s < ns) SQ_STAGE(lA0, lB0, lA1, lB1)
#undef SQ_STAGE
    __builtin_amdgcn_s_waitcnt(0x0070);     // vmcnt(0) lgkmcnt(0): no DMA into LDS outlives the loop

    // This tile's scales, loaded before the next tile's DMAs so that the
    // epilogue waits for these loads only (a bias is read in the epilogue).
    const int cm0 = m0, cn0 = n0;
    float xsv[TI], wv[TJN][4];
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int m = min(cm0 + wm + 16 * i + (lane & 15), M - 1);
      xsv[i] = (YDT == SQ_DT_I32) ? 0.0f : xs[m];
    }
#pragma unroll
    for (int j = 0; j < TJN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int nn = min(cn0 + wn + 16 * j + 4 * (lane >> 4) + r, N - 1);
        wv[j][r] = (YDT == SQ_DT_I32) ? 0.0f : ws[nn];
      }

    // Every wave is done reading the ring: the next tile's first two stages
    // go out now and land while this tile's outputs are written.
    stage_barrier();
    const int vn = v + static_cast<int>(gridDim.x);
    const bool more = vn < ntiles;
    if (more) {
      setup(vn);
      prologue();
    }

    // Epilogue: lane holds acc[m = .. + lane % 16][n = .. + 4 (lane / 16) + r].
    if constexpr (YDT == SQ_DT_F16 || YDT == SQ_DT_BF16) {
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int m = cm0 + wm + 16 * i + (lane & 15);
#pragma unroll
        for (int j = 0; j + 1 < TJN; j += 2)
          store8_pair<YDT>(y, M, N, m, cn0 + wn + 16 * j, acc[i][j], acc[i][j + 1], xsv[i], wv[j], wv[j + 1], bias,
                           lane);
        if constexpr (TJN % 2 == 1) {                   // the odd last tile, four outputs per lane
          const int n = cn0 + wn + 16 * (TJN - 1) + 4 * (lane >> 4);
          if (m < M && n < N) store4_pre<YDT>(y, N, m, n, acc[i][TJN - 1], xsv[i], wv[TJN - 1], bias);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int m = cm0 + wm + 16 * i + (lane & 15);
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < TJN; ++j) {
          const int n = cn0 + wn + 16 * j + 4 * (lane >> 4);
          if (n < N) store4_pre<YDT>(y, N, m, n, acc[i][j], xsv[i], wv[j], bias);
        }
      }
    }
    if (!more) break;
    v = vn;
  }
}

// ----------------------------------------------------------------------------- FP8 (OCP E4M3) tiled kernel

// FP8 operands through the same tile, DMA ring, swizzle and XCD mapping as
// k_gemm_tile, multiplied by v_mfma_scale_f32_16x16x128_f8f6f4 (format 0 =
// E4M3 for both operands, block scales 2^0) into binary32 accumulators. One
// MFMA takes a whole 128-byte stage: lane group g supplies the stage's K bytes
// 16g .. 16g+15 and 64+16g .. 64+16g+15 of its row for both operands (the
// chunks the INT8 kernel reads for its two K steps), so every product pairs
// the same K index. Requires K % 128 == 0.
//
// A stage's fragments (8 A and 4 B blocks of 32 bytes per lane, 96 VGPRs)
// cannot be double-buffered beside the 128 accumulator VGPRs, so the stage
// keeps its B blocks and streams A one row block ahead of the MFMAs: while
// the four MFMAs of block i run, block i+1 is read. After the last block's
// MFMAs are issued the wave waits for stage s+1 (the only DMA in flight) and
// for its own reads of stage s, passes the barrier (every wave is then done
// with stage s's buffer, and stage s+1 is visible), refills that buffer with
// stage s+2, and reads stage s+1's B blocks and first A block while those
// MFMAs drain. Issue indices are clamped to the last stage; the final issues
// and reads are harmless reloads.
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v8i lds_frag8(const int8_t* base, int off0, int off1) {
  const v4i lo = *reinterpret_cast<const v4i*>(base + off0);
  const v4i hi = *reinterpret_cast<const v4i*>(base + off1);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Four MFMAs of A block i against the stage's B blocks, while block i+1 is read
// (the read goes out first, then the MFMAs, in that order).
template <int TJN>
__device__ __forceinline__ void fp8_block(v4f (&acc)[TJN], const v8i& a, const v8i (&fb)[TJN]) {
#pragma unroll
  for (int j = 0; j < TJN; ++j)
    acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fb[j], a, acc[j], 0, 0, 0, 127, 0, 127);
}

template <int YDT, int TJN = 4>
__global__ __launch_bounds__(512, 1) void k_gemm_tile_fp8(const uint8_t* __restrict__ xq, const float* __restrict__ xs,
                                                          const uint8_t* __restrict__ wq, const float* __restrict__ ws,
                                                          const float* __restrict__ bias, void* __restrict__ y, int M,
                                                          int N, int K, int tiles_m, int tiles_n, int group) {
  __shared__ __attribute__((aligned(1024))) int8_t lA0[kStage2Bytes];
  __shared__ __attribute__((aligned(1024))) int8_t lA1[kStage2Bytes];
  __shared__ __attribute__((aligned(1024))) int8_t lB0[kStage2Bytes];
  __shared__ __attribute__((aligned(1024))) int8_t lB1[kStage2Bytes];

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ntiles = tiles_m * tiles_n;
  // persistent over tiles b, b + G, ..., as k_gemm_tile
  int m0 = 0, n0 = 0;
  uint32_t a_off[kDma2PerWave], b_off[TJN];
  __amdgpu_buffer_rsrc_t ra, rb;
  auto setup = [&](int v) {
    int tm, tn;
    map_tile(v, ntiles, tiles_m, group, tm, tn);
    m0 = tm * kTile;
    n0 = tn * (64 * TJN);
    int ln;                                         // the lane id read afresh, as in k_gemm_tile
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
#pragma unroll
    for (int i = 0; i < kDma2PerWave; ++i) {
      const int r = (wid * kDma2PerWave + i) * 8 + (ln >> 3);
      const int c = (ln & 7) ^ swz2(r);
      a_off[i] = static_cast<uint32_t>(min(m0 + r, M - 1) - m0) * static_cast<uint32_t>(K) + 16u * c;
    }
#pragma unroll
    for (int i = 0; i < TJN; ++i) {
      const int r = (wid * TJN + i) * 8 + (ln >> 3);
      const int c = (ln & 7) ^ swz2(r);
      b_off[i] = static_cast<uint32_t>(min(n0 + r, N - 1) - n0) * static_cast<uint32_t>(K) + 16u * c;
    }
    ra = make_rsrc(xq + static_cast<int64_t>(m0) * K);
    rb = make_rsrc(wq + static_cast<int64_t>(n0) * K);
  };
  const int wm = (wid & 1) * 128, wn = (wid >> 1) * (16 * TJN);
  const int rra = wm + (lane & 15), rrb = wn + (lane & 15);
  int a_rd[2], b_rd[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int c = 4 * t + (lane >> 4);
    a_rd[t] = rra * kSlice2 + 16 * (c ^ swz2(rra));
    b_rd[t] = rrb * kSlice2 + 16 * (c ^ swz2(rrb));
  }

  const int ns = K / kSlice2;
  const int last = (ns - 1) * kSlice2;
  auto prologue = [&]() {
    issue_rows2<kDma2PerWave>(ra, lA0, a_off, 0, wid);
    issue_rows2<TJN>(rb, lB0, b_off, 0, wid);
    memory_opaque();
    issue_rows2<kDma2PerWave>(ra, lA1, a_off, min(kSlice2, last), wid);
    issue_rows2<TJN>(rb, lB1, b_off, min(kSlice2, last), wid);
  };
  int v = blockIdx.x;
  setup(v);
  prologue();

  for (;;) {
    v4f acc[TI][TJN];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJN; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    // stage 0 landed: at most stage 1's 4 + TJN DMA instructions outstanding (see k_gemm_tile)
    constexpr int kStageDma = kDma2PerWave + TJN;
    __builtin_amdgcn_s_waitcnt((kStageDma & 15) | ((kStageDma >> 4) << 14) | 0x0F70);
    stage_barrier();
    v8i fb[TJN], a_cur;
    {
      // in asm, as in k_gemm_tile: both K halves of the B blocks and of A block 0
      uint32_t addr[2 * TJN + 2];
      v4i r[2 * TJN + 2];
#pragma unroll
      for (int j = 0; j < TJN; ++j) {
        addr[2 * j] = lds_addr(lB0) + j * 16 * kSlice2 + b_rd[0];
        addr[2 * j + 1] = lds_addr(lB0) + j * 16 * kSlice2 + b_rd[1];
      }
      addr[2 * TJN] = lds_addr(lA0) + a_rd[0];
      addr[2 * TJN + 1] = lds_addr(lA0) + a_rd[1];
      lds_read_frags(r, addr);
#pragma unroll
      for (int j = 0; j < TJN; ++j) fb[j] = __builtin_shufflevector(r[2 * j], r[2 * j + 1], 0, 1, 2, 3, 4, 5, 6, 7);
      a_cur = __builtin_shufflevector(r[2 * TJN], r[2 * TJN + 1], 0, 1, 2, 3, 4, 5, 6, 7);
    }

#define SQ_FP8_STAGE(LA, LB, LA_NXT, LB_NXT)                                                              \
  {                                                                                                      \
    _Pragma("unroll") for (int i = 0; i + 1 < TI; ++i) {                                                 \
      const v8i a_nxt = lds_frag8(LA + (i + 1) * 16 * kSlice2, a_rd[0], a_rd[1]);                        \
      fp8_block(acc[i], a_cur, fb);                                                                      \
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0); /* the two LDS reads of block i+1 */            \
      __builtin_amdgcn_sched_group_barrier(0x008, TJN, 0); /* then block i's MFMAs */                    \
      a_cur = a_nxt;                                                                                     \
    }                                                                                                    \
    fp8_block(acc[TI - 1], a_cur, fb);                                                                   \
    __builtin_amdgcn_sched_barrier(0);                                                                   \
    __builtin_amdgcn_s_waitcnt(0x0070); /* vmcnt(0) lgkmcnt(0): stage s+1 landed, stage s reads done */ \
    stage_barrier();                                                                                     \
    const int kn = min((s + 2) * kSlice2, last);                                                          \
    issue_rows2<kDma2PerWave>(ra, LA, a_off, kn, wid);                                                   \
    issue_rows2<TJN>(rb, LB, b_off, kn, wid);                                                            \
    _Pragma("unroll") for (int j = 0; j < TJN; ++j)                                                      \
      fb[j] = lds_frag8(LB_NXT + j * 16 * kSlice2, b_rd[0], b_rd[1]);                                    \
    a_cur = lds_frag8(LA_NXT, a_rd[0], a_rd[1]);                                                         \
    __builtin_amdgcn_sched_barrier(0);                                                                   \
    ++s;                                                                                                 \
  }
    int s = 0;
    for (; s + 2 <= ns;) {
      SQ_FP8_STAGE(lA0, lB0, lA1, lB1)
      SQ_FP8_STAGE(lA1, lB1, lA0, lB0)
    }
    if (s < ns) SQ_FP8_STAGE(lA0, lB0, lA1, lB1)
#undef SQ_FP8_STAGE
    __builtin_amdgcn_s_waitcnt(0x0070);     // no DMA into LDS outlives the loop

    // this tile's scales before the next tile's DMAs, then the epilogue (as k_gemm_tile)
    const int cm0 = m0, cn0 = n0;
    float xsv[TI], wv[TJN][4];
#pragma unroll
    for (int i = 0; i < TI; ++i) xsv[i] = xs[min(cm0 + wm + 16 * i + (lane & 15), M - 1)];
#pragma unroll
    for (int j = 0; j < TJN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) wv[j][r] = ws[min(cn0 + wn + 16 * j + 4 * (lane >> 4) + r, N - 1)];
    stage_barrier();
    const int vn = v + static_cast<int>(gridDim.x);
    const bool more = vn < ntiles;
    if (more) {
      setup(vn);
      prologue();
    }
    if constexpr (YDT == SQ_DT_F16 || YDT == SQ_DT_BF16) {
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int m = cm0 + wm + 16 * i + (lane & 15);
#pragma unroll
        for (int j = 0; j + 1 < TJN; j += 2)
          store8_pair<YDT, v4f>(y, M, N, m, cn0 + wn + 16 * j, acc[i][j], acc[i][j + 1], xsv[i], wv[j], wv[j + 1],
                                bias, lane);
        if constexpr (TJN % 2 == 1) {                   // the odd last tile, four outputs per lane
          const int n = cn0 + wn + 16 * (TJN - 1) + 4 * (lane >> 4);
          if (m < M && n < N) store4_pre<YDT, v4f>(y, N, m, n, acc[i][TJN - 1], xsv[i], wv[TJN - 1], bias);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int m = cm0 + wm + 16 * i + (lane & 15);
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < TJN; ++j) {
          const int n = cn0 + wn + 16 * j + 4 * (lane >> 4);
          if (n < N) store4_pre<YDT, v4f>(y, N, m, n, acc[i][j], xsv[i], wv[j], bias);
        }
      }
    }
    if (!more) break;
    v = vn;
  }
}

// ----------------------------------------------------------------------------- decode helpers

// Decode shapes (M <= 128) are bound by streaming wq once from HBM. HBM and the
// L2 serve a wave's load best when it covers whole 128-byte lines: a load in
// the MFMA register layout (16 rows x 64 bytes) reaches about 2/3 of the rate
// of one that covers 4 or 8 rows x 256 or 128 bytes, so the decode kernels
// never load weights in the MFMA layout directly.
constexpr int kDecWaves = 4;
// Up to this many tokens the weight-streaming kernels run the GEMM. From 65 to
// 128 tokens the 256-row prefill tile would leave half of every tile and most
// CUs idle (36-144 tiles at N = 4096-36864): measured at K = 9216 with rotating
// weights, eight token tiles per strip took 33-36 us against 72-74 us at
// N = 4096 and 9216, and 82-88 against 105-110 us at N = 36864.
constexpr int kDecMaxTokens = 128;
// Buffer-load cache policy for the decode weight stream, read exactly once:
// non-temporal. Measured on the 1-token GEMV, N = 36864: 6.5 against 5.8 TB/s.
constexpr int kStreamPolicy = 2;
// s_waitcnt immediate: vmcnt(n), lgkmcnt(0), expcnt not waited on.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0070; }

// Buffer resource over `bytes` bytes at `base`; loads past the end return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_n(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}

// ----------------------------------------------------------------------------- decode kernel, 128-byte segments

// The decode kernel with the prefill kernel's LDS layout: K in 128-byte
// segments (two MFMA K steps), operand tiles of 16 rows x 128 bytes (row r at
// r * 128, chunk c at slot c ^ swz2(r)), and DMA blocks of 8 rows x 128 bytes,
// two per tile. A workgroup owns a strip of ch <= 16 NT channels (a multiple
// of 4) in NT channel tiles (up to 9: a 144-channel strip, so 36864 channels
// make exactly 256 workgroups and each xq segment serves NT weight tiles);
// rows past the strip read zeros and are not stored. Every wave works on every segment, on its own
// block of channel tiles x token tiles (1, 2 or 4 token groups times 4, 2 or
// 1 channel groups, whichever leaves the busiest wave the least MFMA and LDS
// work), and stores its own outputs: no partial sums pass between waves. Segments go
// through an R-stage ring.
//
// INT8: two v_mfma_i32_16x16x64_i8 per tile and segment, one per 64-byte half
// (the second skipped on an odd last K step, whose bytes belong to the next
// row). FP8 (E4M3 codes, K % 128 == 0): one v_mfma_scale_f32_16x16x128_f8f6f4
// takes the whole segment (K bytes 16g .. 16g+15 and 64+16g .. 64+16g+15 of a
// row for lane group g, as in the prefill kernel), into binary32 accumulators.
// Token groups of the decode wave grid (1, 2 or 4; the channel groups take the
// rest of the four waves). The busiest wave's cost per segment is weighed as
// 2 x its tiles (two INT8 MFMAs or one FP8 MFMA each) + its fragment-tile
// reads from LDS (one per channel tile and per token tile), and the lowest
// cost wins, the fewest token groups on a tie. Measured at K = 9216: with three
// channel and three token tiles one token group beat a 2 x 2 grid by 13%; with
// nine channel and four token tiles the 2 x 2 grid beat four token groups by 1%.
constexpr int dec_token_groups(int nt, int mt) {
  int best = 1, best_cost = 1 << 30;
  for (int wu = 1; wu <= kDecWaves; wu *= 2) {
    const int nc = (nt + kDecWaves / wu - 1) / (kDecWaves / wu), mu = (mt + wu - 1) / wu;
    if (2 * nc * mu + nc + mu < best_cost) {
      best = wu;
      best_cost = 2 * nc * mu + nc + mu;
    }
  }
  return best;
}
constexpr int kDecNowhere = 0x40000000;               // a buffer offset past every operand: loads return zeros
constexpr int kDec2Seg = 128;
constexpr int kDec2Tile = 16 * kDec2Seg;             // LDS bytes of one 16-row operand tile

template <int NT, int MT, int R, int YDT, bool FP8 = false>
__global__ __launch_bounds__(64 * kDecWaves) void k_gemm_decode(const int8_t* __restrict__ xq,
                                                                const float* __restrict__ xs,
                                                                const int8_t* __restrict__ wq,
                                                                const float* __restrict__ ws,
                                                                const float* __restrict__ bias, void* __restrict__ y,
                                                                int M, int N, int K, int ch) {
  static_assert(R >= 3 && R <= 8, "ring depth");
  constexpr int kTiles = NT + MT;
  constexpr int kWPer = (2 * NT + kDecWaves - 1) / kDecWaves;     // weight DMA blocks per wave per segment
  constexpr int kXPer = (2 * MT + kDecWaves - 1) / kDecWaves;     // token DMA blocks per wave per segment
  constexpr int kPerWave = kWPer + kXPer;                          // DMA instructions per wave per segment
  constexpr bool kSink = (2 * NT) % kDecWaves != 0 || (2 * MT) % kDecWaves != 0;   // padding DMAs need a sink
  constexpr int kStage = kTiles * kDec2Tile + (kSink ? 1024 : 0);
  // wave grid: WU token groups x (kDecWaves / WU) channel groups, NC x MU tiles per wave
  constexpr int WU = dec_token_groups(NT, MT);
  constexpr int NC = (NT + kDecWaves / WU - 1) / (kDecWaves / WU);
  constexpr int MU = (MT + WU - 1) / WU;
  __shared__ __attribute__((aligned(1024))) int8_t st0[kStage];
  __shared__ __attribute__((aligned(1024))) int8_t st1[kStage];
  __shared__ __attribute__((aligned(1024))) int8_t st2[kStage];
  __shared__ __attribute__((aligned(1024))) int8_t st3[R > 3 ? kStage : 16];
  __shared__ __attribute__((aligned(1024))) int8_t st4[R > 4 ? kStage : 16];
  __shared__ __attribute__((aligned(1024))) int8_t st5[R > 5 ? kStage : 16];
  __shared__ __attribute__((aligned(1024))) int8_t st6[R > 6 ? kStage : 16];
  __shared__ __attribute__((aligned(1024))) int8_t st7[R > 7 ? kStage : 16];
  auto stage = [&](auto k) -> int8_t* {
    constexpr int i = decltype(k)::value;
    if constexpr (i == 0) return st0;
    else if constexpr (i == 1) return st1;
    else if constexpr (i == 2) return st2;
    else if constexpr (i == 3) return st3;
    else if constexpr (i == 4) return st4;
    else if constexpr (i == 5) return st5;
    else if constexpr (i == 6) return st6;
    else return st7;
  };

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * ch;                                  // ch <= 16 NT channels, a multiple of 4
  const int rows_w = min(ch, N - n0);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc_n(wq + static_cast<int64_t>(n0) * K, static_cast<uint32_t>(rows_w * K));
  const __amdgpu_buffer_rsrc_t rx = make_rsrc_n(xq, static_cast<uint32_t>(M * K));
  const int steps = K >> 6;
  const int segs = (steps + 1) >> 1;

  // Weight blocks b = wid + 4 i (tile b / 2, rows 8 (b % 2) .. +8 of it), then
  // token blocks likewise; blocks past the operand's count load nothing into
  // the sink. (Offsets are recomputed per issue: per-wave tables indexed inside
  // the lambda make the host compiler drop the kernel's launch stub.)
  const int rr = lane >> 3;                                     // row within a DMA block
  const uint32_t lane_src0 = static_cast<uint32_t>(rr * K + 16 * ((lane & 7) ^ swz2(rr)));
  const uint32_t lane_src1 = static_cast<uint32_t>((8 + rr) * K + 16 * ((lane & 7) ^ swz2(8 + rr)));
  auto issue = [&](auto k, int seg) {
    const int so = seg < segs ? seg * kDec2Seg : kDecNowhere;
    int8_t* stg = stage(k);
#pragma unroll
    for (int i = 0; i < kWPer + kXPer; ++i) {
      const bool w = i < kWPer;
      const int b = wid + kDecWaves * (w ? i : i - kWPer);
      const bool real = b < 2 * (w ? NT : MT);
      const int tile = real ? b >> 1 : 0, half = b & 1;
      const uint32_t src = static_cast<uint32_t>(16 * tile * K) + (half ? lane_src1 : lane_src0);
      const int dst = real ? ((w ? 0 : NT) + tile) * kDec2Tile + half * 1024 : kTiles * kDec2Tile;
      if (w)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_ptr_t)(stg + dst), 16, src, real ? so : kDecNowhere, 0,
                                                 kStreamPolicy);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr_t)(stg + dst), 16, src, real ? so : kDecNowhere, 0, 0);
    }
  };

  // compute share: channel tiles [c0, c0 + NC) x token tiles [u0, u0 + MU) of
  // every segment (clipped to NT, MT); lane group g reads its 16 bytes of
  // each 64-byte half of the segment's rows
  using AccV = std::conditional_t<FP8, v4f, v4i>;
  const int r16 = lane & 15;
  const int frag_lo = r16 * kDec2Seg + 16 * ((lane >> 4) ^ swz2(r16));
  const int frag_hi = r16 * kDec2Seg + 16 * ((4 + (lane >> 4)) ^ swz2(r16));
  const int c0 = (wid / WU) * NC, u0 = (wid % WU) * MU;
  AccV acc[NC][MU];
#pragma unroll
  for (int j = 0; j < NC; ++j)
#pragma unroll
    for (int u = 0; u < MU; ++u) acc[j][u] = AccV{0, 0, 0, 0};

#define SQ_DEC_PRO(I) \
  if constexpr (I < R - 1) { issue(std::integral_constant<int, I>{}, I); memory_opaque(); }
  SQ_DEC_PRO(0) SQ_DEC_PRO(1) SQ_DEC_PRO(2) SQ_DEC_PRO(3) SQ_DEC_PRO(4) SQ_DEC_PRO(5) SQ_DEC_PRO(6)
#undef SQ_DEC_PRO

  auto step = [&](auto k, int seg) {
    constexpr int kk = decltype(k)::value;
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((R - 2) * kPerWave));
    stage_barrier();
    issue(std::integral_constant<int, (kk + R - 1) % R>{}, seg + R - 1);
    if (c0 < NT && u0 < MT) {                                    // uniform: a wave past the tiles only waits
      const uint32_t b = lds_addr(stage(k));
      uint32_t addr[2 * (NC + MU)];
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        const uint32_t tb = b + min(c0 + j, NT - 1) * kDec2Tile;
        addr[2 * j] = tb + frag_lo;
        addr[2 * j + 1] = tb + frag_hi;
      }
#pragma unroll
      for (int u = 0; u < MU; ++u) {
        const uint32_t tb = b + (NT + min(u0 + u, MT - 1)) * kDec2Tile;
        addr[2 * (NC + u)] = tb + frag_lo;
        addr[2 * (NC + u) + 1] = tb + frag_hi;
      }
      v4i f[2 * (NC + MU)];
      lds_read_frags(f, addr);
      if constexpr (FP8) {
#pragma unroll
        for (int j = 0; j < NC; ++j) {
          const v8i fw = __builtin_shufflevector(f[2 * j], f[2 * j + 1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
          for (int u = 0; u < MU; ++u) {
            const v8i fx = __builtin_shufflevector(f[2 * (NC + u)], f[2 * (NC + u) + 1], 0, 1, 2, 3, 4, 5, 6, 7);
            acc[j][u] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fw, fx, acc[j][u], 0, 0, 0, 127, 0, 127);
          }
        }
      } else {
        const bool two = 2 * seg + 1 < steps;                    // uniform: an odd last K step has one half
#pragma unroll
        for (int j = 0; j < NC; ++j)
#pragma unroll
          for (int u = 0; u < MU; ++u) {
            acc[j][u] = __builtin_amdgcn_mfma_i32_16x16x64_i8(f[2 * j], f[2 * (NC + u)], acc[j][u], 0, 0, 0);
            if (two)
              acc[j][u] = __builtin_amdgcn_mfma_i32_16x16x64_i8(f[2 * j + 1], f[2 * (NC + u) + 1], acc[j][u], 0, 0, 0);
          }
      }
    }
  };
  int base = 0;
  for (; base + R <= segs; base += R) {
#define SQ_DEC_STEP(I) \
  if constexpr (I < R) step(std::integral_constant<int, I>{}, base + I);
    SQ_DEC_STEP(0) SQ_DEC_STEP(1) SQ_DEC_STEP(2) SQ_DEC_STEP(3) SQ_DEC_STEP(4) SQ_DEC_STEP(5) SQ_DEC_STEP(6)
    SQ_DEC_STEP(7)
#undef SQ_DEC_STEP
  }
#define SQ_DEC_TAIL(I) \
  if constexpr (I < R - 1) { if (base + I < segs) step(std::integral_constant<int, I>{}, base + I); }
  SQ_DEC_TAIL(0) SQ_DEC_TAIL(1) SQ_DEC_TAIL(2) SQ_DEC_TAIL(3) SQ_DEC_TAIL(4) SQ_DEC_TAIL(5) SQ_DEC_TAIL(6)
#undef SQ_DEC_TAIL

  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));                    // no DMA into LDS outlives the loop
  // every wave stores its own channel x token tiles
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    if (c0 + j >= NT) continue;                                    // uniform
#pragma unroll
    for (int u = 0; u < MU; ++u) {
      if (u0 + u >= MT) continue;                                  // uniform
      const int m = 16 * (u0 + u) + (lane & 15);
      const int n = n0 + 16 * (c0 + j) + 4 * (lane >> 4);
      if (m < M && n < n0 + rows_w) store4<YDT>(y, N, m, n, acc[j][u], (YDT == SQ_DT_I32) ? 0.0f : xs[m], ws, bias);
    }
  }
}

// ----------------------------------------------------------------------------- GEMV kernel (up to 8 tokens)

// y[m, n] for one output, same rounding as store4.
template <int YDT>
__device__ __forceinline__ void store1(void* __restrict__ y, int N, int m, int n, int acc, float xs,
                                       const float* __restrict__ ws, const float* __restrict__ bias) {
  const int64_t off = static_cast<int64_t>(m) * N + n;
  if constexpr (YDT == SQ_DT_I32) {
    static_cast<int*>(y)[off] = acc;
  } else {
    float t = mul_rn(mul_rn(static_cast<float>(acc), xs), ws[n]);
    if (bias) t = add_rn(t, bias[n]);
    if constexpr (YDT == SQ_DT_F32) static_cast<float*>(y)[off] = t;
    else static_cast<uint16_t*>(y)[off] = static_cast<uint16_t>(YDT == SQ_DT_F16 ? f32_to_f16_rne(t) : f32_to_bf16_rne(t));
  }
}

// Decode with a handful of tokens on the vector ALUs: the weight stream is the
// whole cost, and a load of 4 rows x 256 bytes (whole lines) per wave
// instruction streams at the full HBM rate with no LDS staging or barriers.
// A workgroup owns 16 channels and its four waves split K; lane l holds the
// 16-byte K chunk l % 16 of rows 4 i + l / 16 (i = 0..3) of each 256-byte
// segment, multiplies it against the same chunk of each token with
// v_dot4_i32_i8 (int32 accumulation, exact), and keeps 4 x MM partial sums.
// At the end the 16 lanes of a row are summed by DPP and the four waves
// through LDS. Integer sums are exact, so the order does not matter.
template <int MM, int U, int YDT>
__global__ __launch_bounds__(256) void k_gemv(const int8_t* __restrict__ xq, const float* __restrict__ xs,
                                              const int8_t* __restrict__ wq, const float* __restrict__ ws,
                                              const float* __restrict__ bias, void* __restrict__ y, int M, int N,
                                              int K) {
  __shared__ int red[kDecWaves][16][MM];
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * 16;
  const int rows_w = min(16, N - n0);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc_n(wq + static_cast<int64_t>(n0) * K, static_cast<uint32_t>(rows_w * K));
  const __amdgpu_buffer_rsrc_t rx = make_rsrc_n(xq, static_cast<uint32_t>(M * K));
  const int c = lane & 15, g = lane >> 4;
  const int segs = (K + 255) >> 8;
  const int q = (segs + kDecWaves - 1) / kDecWaves;
  const int s0 = wid * q, s1 = min(s0 + q, segs);
  int acc[4][MM];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int m = 0; m < MM; ++m) acc[i][m] = 0;

  auto seg_step = [&](int s) {
    // chunks past K (only in a last, partial segment) load zeros
    const bool ok = s * 256 + 16 * c < K;
    v4i w[4], x[MM];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(
                                         rw, ok ? static_cast<uint32_t>((4 * i + g) * K + 16 * c) : kDecNowhere,
                                         s * 256, kStreamPolicy));
#pragma unroll
    for (int m = 0; m < MM; ++m)
      x[m] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(
                                         rx, ok ? static_cast<uint32_t>(m * K + 16 * c) : kDecNowhere, s * 256, 0));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int m = 0; m < MM; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][m] = __builtin_amdgcn_sdot4(w[i][j], x[m][j], acc[i][m], false);
  };
  int s = s0;
  for (; s + U <= s1; s += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) seg_step(s + u);
  }
  for (; s < s1; ++s) seg_step(s);

  // sum the 16 lanes of each row (one DPP row), then the four waves
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int m = 0; m < MM; ++m) {
      int v = acc[i][m];
      v += dpp_move<kDppXor1>(v);
      v += dpp_move<kDppXor2>(v);
      v += dpp_move<kDppHalfMirror>(v);
      v += dpp_move<kDppMirror>(v);
      if (c == 0) red[wid][4 * i + g][m] = v;
    }
  __syncthreads();
  const int t = threadIdx.x;
  if (t < 16 * MM) {
    const int row = t & 15, m = t >> 4;
    const int n = n0 + row;
    if (m < M && n < N) {
      int v = 0;
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) v += red[w][row][m];
      store1<YDT>(y, N, m, n, v, (YDT == SQ_DT_I32) ? 0.0f : xs[m], ws, bias);
    }
  }
}

// ----------------------------------------------------------------------------- row GEMV (1-2 tokens, K <= 9216)

// Decode with a handful of tokens, read the way a plain streaming kernel reads:
// each wave takes whole weight rows, one at a time, and each of its load
// instructions covers 1 KiB of one row (lane l: bytes 16 l .. 16 l + 15 of each
// 1024-byte chunk), so the weight stream is contiguous per instruction. Every
// lane holds its 16-byte K chunks of all MM tokens in registers for the whole
// kernel (CH chunks per token: K <= 1024 CH; chunks past K and tokens past M
// are zeros), multiplies them against the row with v_dot4_i32_i8 (int32,
// exact), and the row's 64 lane sums are added by DPP inside each 16-lane row
// and across the four rows through scalar reads. The next row's loads are in
// flight while a row is reduced. Waves take rows gw, gw + GW, ... (GW = all
// waves of the grid). Lane t < M stores token t's output.
// Row n's chunks into w; a row past the end (valid false) gets a zero-length
// resource: its loads return zeros without touching memory, so the loads are
// issued unconditionally and the wait counts stay exact.
template <int MM, int CH>
__device__ __forceinline__ void gemv_row_load(const int8_t* __restrict__ wq, int64_t n, bool valid, int K, int lane,
                                              v4i (&w)[CH]) {
  const __amdgpu_buffer_rsrc_t rw = make_rsrc_n(wq + n * K, valid ? static_cast<uint32_t>(K) : 0u);
#pragma unroll
  for (int c = 0; c < CH; ++c)
    w[c] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rw, static_cast<uint32_t>(1024 * c + 16 * lane),
                                                                        0, kStreamPolicy));
}

template <int MM, int CH, int YDT>
__device__ __forceinline__ void gemv_row_finish(const v4i (&w)[CH], const v4i (&x)[MM][CH], int64_t n, int lane,
                                                int M, int N, float xs_lane, const float* __restrict__ ws,
                                                const float* __restrict__ bias, void* __restrict__ y) {
  int acc[MM];
#pragma unroll
  for (int t = 0; t < MM; ++t) {
    acc[t] = 0;
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[t] = __builtin_amdgcn_sdot4(w[c][j], x[t][c][j], acc[t], false);
  }
  int mine = 0;
#pragma unroll
  for (int t = 0; t < MM; ++t) {
    int v = acc[t];
    v += dpp_move<kDppXor1>(v);
    v += dpp_move<kDppXor2>(v);
    v += dpp_move<kDppHalfMirror>(v);
    v += dpp_move<kDppMirror>(v);
    const int total = (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
                      (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
    if (lane == t) mine = total;
  }
  if (lane < M) store1<YDT>(y, N, lane, static_cast<int>(n), mine, xs_lane, ws, bias);
}

template <int MM, int CH, int YDT>
__global__ __launch_bounds__(256) void k_gemv_rows(const int8_t* __restrict__ xq, const float* __restrict__ xs,
                                                   const int8_t* __restrict__ wq, const float* __restrict__ ws,
                                                   const float* __restrict__ bias, void* __restrict__ y, int M, int N,
                                                   int K) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));   // uniform
  const int nw = gridDim.x * 4;
  // this lane's K chunks of every token (zeros past K or past M)
  const __amdgpu_buffer_rsrc_t rx = make_rsrc_n(xq, static_cast<uint32_t>(M * K));
  v4i x[MM][CH];
#pragma unroll
  for (int t = 0; t < MM; ++t)
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int k = 1024 * c + 16 * lane;
      const uint32_t off = (t < M && k < K) ? static_cast<uint32_t>(t * K + k) : kDecNowhere;
      x[t][c] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
    }
  const float xs_lane = (YDT != SQ_DT_I32 && lane < M) ? xs[lane] : 0.0f;   // lane t stores token t
  int64_t n = gw;
  if (n >= N) return;
  v4i wa[CH], wb[CH];
  gemv_row_load<MM, CH>(wq, n, true, K, lane, wa);
  for (;;) {
    const int64_t n1 = n + nw;
    gemv_row_load<MM, CH>(wq, n1 < N ? n1 : n, n1 < N, K, lane, wb);
    gemv_row_finish<MM, CH, YDT>(wa, x, n, lane, M, N, xs_lane, ws, bias, y);
    if (n1 >= N) break;
    const int64_t n2 = n1 + nw;
    gemv_row_load<MM, CH>(wq, n2 < N ? n2 : n1, n2 < N, K, lane, wa);
    gemv_row_finish<MM, CH, YDT>(wb, x, n1, lane, M, N, xs_lane, ws, bias, y);
    if (n2 >= N) break;
    n = n2;
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));        // the last (empty) loads land before the wave ends
}

namespace {

// The row GEMV's grid: two workgroups (8 waves) per CU, within what fits, at
// most one wave per row. Measured at K = 9216 with rotating weights: one
// workgroup per CU and two gave 15.2-15.5 us for N = 9216 and 1-2 tokens,
// four 15.0-16.5; grids that are not a multiple of the CU count (341, 682)
// were 1-2 us slower (uneven per-CU load). Without the next row's loads in
// flight two tokens took 16.2-27 us.
template <int MM, int CH, int YDT>
hipError_t launch_rows(const GemmArgs& g, hipStream_t st) {
  auto kern = k_gemv_rows<MM, CH, YDT>;
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kern),
                                                                        256, 0);
  if (e != hipSuccess) return e;
  const int cap = max(1, cus * min(max(per_cu, 1), 2));
  const int grid = min((g.N + 3) / 4, cap);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, st, g.xq, g.x_scale, g.wq, g.w_scale, g.bias, g.y, g.M, g.N,
                     g.K);
  return hipGetLastError();
}

// Decode shapes (M <= 128). INT8 with 1-2 tokens, K <= 9216 and N < 16384: the
// row GEMV (k_gemv_rows, 14.7-15.6 us at N = 9216 against 15.8-16.8 for the
// MFMA kernel; at N = 36864 it trails k_gemv by 1-2%; with 4 tokens, 234
// VGPRs, it took 16.6 us against the MFMA kernel's 16.0). INT8 with up to 4
// tokens at N >= 16384: the vector-ALU GEMV, 16 channels per workgroup (6.8
// TB/s at N = 36864, where the MFMA kernel reaches 6.5). Otherwise the MFMA
// decode kernel (gfx950 has no FP8 dot product on the vector ALUs, so FP8
// always takes it) with up to 9 channel tiles per workgroup at N >= 16384,
// so that each token segment serves many weight tiles, and 3 below. Each
// workgroup takes its share of the channels, N / CUs rounded up to a multiple
// of 4, within 48 (3 tiles) or 48-144 (9 tiles), so that every CU streams
// weights: 36 channels at N = 9216 (the third tile has 4 real rows; rows past
// the strip read zeros without touching memory), 144 at N = 36864. Against
// fixed 48- and 144-channel strips (192 workgroups at N = 9216, 114 at 16384,
// 143 at 20480) that took 4-64 tokens at N = 9216 from 17.0-28.9 to 16.8-27.8
// us (32 tokens: 21.7 to 19.4), N = 16384 from 32.8 / 41.6 / 49.6 to 30.4 /
// 35.6 / 45.4 us at 8 / 32 / 64 tokens (K = 8192) and 16 tokens at N = 20480
// from 41.6 to 34.3 us; 48-channel strips had beaten 64-channel ones (144
// workgroups) by 10-11% at 8-32 tokens. Measured on K = 9216 unless stated.
template <int YDT, bool FP8>
hipError_t launch_decode(const GemmArgs& g, hipStream_t st) {
  const int mt = (g.M + 15) / 16;
  const bool wide = g.N >= 16384;
  int dev = 0, cus = 0;
  if (hipError_t e = hipGetDevice(&dev)) return e;
  if (hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) return e;
  const int per_cu = ((g.N + max(cus, 1) - 1) / max(cus, 1) + 3) & ~3;   // channels per workgroup:
  const int narrow = min(48, max(4, per_cu));                              //   3-tile strips
  const int wch = min(144, max(48, per_cu));                               //   9-tile strips
#define SQ_DECODE(KERN, CH)                                                                                  \
  {                                                                                                          \
    hipLaunchKernelGGL(KERN, dim3((g.N + (CH) - 1) / (CH)), dim3(64 * kDecWaves), 0, st, g.xq, g.x_scale,   \
                       g.wq, g.w_scale, g.bias, g.y, g.M, g.N, g.K, (CH));                                  \
    return hipGetLastError();                                                                                \
  }
#define SQ_GEMV(KERN)                                                                                        \
  {                                                                                                          \
    hipLaunchKernelGGL(KERN, dim3((g.N + 15) / 16), dim3(256), 0, st, g.xq, g.x_scale, g.wq, g.w_scale,     \
                       g.bias, g.y, g.M, g.N, g.K);                                                          \
    return hipGetLastError();                                                                                \
  }
  if (!FP8 && g.M <= 2 && g.K <= 9216 && !wide) {
    if (g.K <= 4096) return g.M == 1 ? launch_rows<1, 4, YDT>(g, st) : launch_rows<2, 4, YDT>(g, st);
    return g.M == 1 ? launch_rows<1, 9, YDT>(g, st) : launch_rows<2, 9, YDT>(g, st);
  }
  if (!FP8 && wide) {
    if (g.M == 1) SQ_GEMV((k_gemv<1, 3, YDT>))
    if (g.M == 2) SQ_GEMV((k_gemv<2, 3, YDT>))
    if (g.M <= 4) SQ_GEMV((k_gemv<4, 2, YDT>))
  }
  if (mt == 1) {
    if (wide) SQ_DECODE((k_gemm_decode<9, 1, 7, YDT, FP8>), wch)
    SQ_DECODE((k_gemm_decode<3, 1, 7, YDT, FP8>), narrow)
  }
  if (mt == 2) {
    if (wide) SQ_DECODE((k_gemm_decode<9, 2, 6, YDT, FP8>), wch)
    SQ_DECODE((k_gemm_decode<3, 2, 6, YDT, FP8>), narrow)
  }
  if (mt == 3) {
    if (wide) SQ_DECODE((k_gemm_decode<9, 3, 5, YDT, FP8>), wch)
    SQ_DECODE((k_gemm_decode<3, 3, 5, YDT, FP8>), narrow)
  }
  if (mt > 4) {                    // 65-128 tokens: eight token tiles, one ring stage fewer to fit LDS
    if (wide) SQ_DECODE((k_gemm_decode<9, 8, 4, YDT, FP8>), wch)
    SQ_DECODE((k_gemm_decode<3, 8, 6, YDT, FP8>), narrow)
  }
  if (wide) SQ_DECODE((k_gemm_decode<9, 4, 5, YDT, FP8>), wch)
  SQ_DECODE((k_gemm_decode<3, 4, 5, YDT, FP8>), narrow)
#undef SQ_DECODE
#undef SQ_GEMV
}

// Grid of a tiled GEMM kernel over ntiles tiles. Up to kPersistWaves tiles per
// resident workgroup, one workgroup per resident slot (a multiple of 8) that
// loops over the tiles: each tile's epilogue then overlaps the next tile's
// first stages instead of a workgroup turnover, which took the K = 4096
// prefill shapes 8-14% faster. Beyond that, one workgroup per tile: the
// looping workgroups drift apart over many tiles, the tiles running at once
// share fewer operand rows in L2, and on 8192 x 81920 x 20480 (40 tiles per
// workgroup) HBM fetch rose from 20.1 to 25.2 GB per launch at the same time,
// where the hardware dispatcher, handing each free CU the next tile, keeps the
// running tiles together.
constexpr int kPersistWaves = 16;
inline hipError_t tile_grid(const void* kernel, int ntiles, int* grid) {
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 512, 0);
  if (e != hipSuccess) return e;
  const int cap = max(8, cus * max(per_cu, 1)) & ~7;
  *grid = (ntiles <= cap || ntiles > kPersistWaves * cap) ? ntiles : cap;
  return hipSuccess;
}

// Tile width for a prefill shape: the width (tiles per wave TJN = 4, 3, 2:
// 256, 192, 128 columns) whose grid costs least, counting each wave of
// resident workgroups at the width's measured time per tile relative to the
// 256-column tile.
constexpr float kTileCost[5] = {0.0f, 0.0f, 0.60f, 0.81f, 1.0f};
inline hipError_t tile_width(int M, int N, int* tjn) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int tiles_m = (M + kTile - 1) / kTile;
  float best = 0.0f;
  *tjn = 4;
  for (int t = 4; t >= 2; --t) {
    const int tiles = tiles_m * ((N + 64 * t - 1) / (64 * t));
    const float cost = static_cast<float>((tiles + cus - 1) / cus) * kTileCost[t];
    if (t == 4 || cost < best) {
      best = cost;
      *tjn = t;
    }
  }
  return hipSuccess;
}

template <int YDT, int TJN>
hipError_t launch_tile(const GemmArgs& g, int tiles_m, int group, hipStream_t st) {
  const int tiles_n = (g.N + 64 * TJN - 1) / (64 * TJN);
  int grid = 0;
  if (hipError_t e = tile_grid(reinterpret_cast<const void*>(k_gemm_tile<YDT, TJN>), tiles_m * tiles_n, &grid))
    return e;
  hipLaunchKernelGGL((k_gemm_tile<YDT, TJN>), dim3(grid), dim3(512), 0, st, g.xq, g.x_scale, g.wq, g.w_scale, g.bias,
                     g.y, g.M, g.N, g.K, tiles_m, tiles_n, group);
  return hipGetLastError();
}

template <int YDT>
hipError_t launch_typed(const GemmArgs& g, hipStream_t st) {
  if (g.M <= kDecMaxTokens) return launch_decode<YDT, false>(g, st);
  const int tiles_m = (g.M + kTile - 1) / kTile;
  const int tiles_n = (g.N + kTile - 1) / kTile;
  const int group = min(tiles_m, 8);
  if (g.K % kSlice2 == 0) {
    int tjn = 4;
    if (hipError_t e = tile_width(g.M, g.N, &tjn)) return e;
    if (tjn == 3) return launch_tile<YDT, 3>(g, tiles_m, group, st);
    if (tjn == 2) return launch_tile<YDT, 2>(g, tiles_m, group, st);
    return launch_tile<YDT, 4>(g, tiles_m, group, st);
  } else
    hipLaunchKernelGGL((k_gemm_tile_k64<YDT>), dim3(tiles_m * tiles_n), dim3(512), 0, st, g.xq, g.x_scale, g.wq,
                       g.w_scale, g.bias, g.y, g.M, g.N, g.K, tiles_m, tiles_n, group);
  return hipGetLastError();
}

}  // namespace

template <int YDT, int TJN>
hipError_t launch_tile_fp8(const GemmArgs& g, int tiles_m, int group, hipStream_t st) {
  const int tiles_n = (g.N + 64 * TJN - 1) / (64 * TJN);
  int grid = 0;
  if (hipError_t e = tile_grid(reinterpret_cast<const void*>(k_gemm_tile_fp8<YDT, TJN>), tiles_m * tiles_n, &grid))
    return e;
  hipLaunchKernelGGL((k_gemm_tile_fp8<YDT, TJN>), dim3(grid), dim3(512), 0, st,
                     reinterpret_cast<const uint8_t*>(g.xq), g.x_scale, reinterpret_cast<const uint8_t*>(g.wq),
                     g.w_scale, g.bias, g.y, g.M, g.N, g.K, tiles_m, tiles_n, group);
  return hipGetLastError();
}

template <int YDT>
hipError_t launch_fp8_typed(const GemmArgs& g, hipStream_t st) {
  if (g.M <= kDecMaxTokens) return launch_decode<YDT, true>(g, st);
  const int tiles_m = (g.M + kTile - 1) / kTile;
  const int group = min(tiles_m, 8);
  int tjn = 4;
  if (hipError_t e = tile_width(g.M, g.N, &tjn)) return e;
  if (tjn == 3) return launch_tile_fp8<YDT, 3>(g, tiles_m, group, st);
  if (tjn == 2) return launch_tile_fp8<YDT, 2>(g, tiles_m, group, st);
  return launch_tile_fp8<YDT, 4>(g, tiles_m, group, st);
}

hipError_t launch_gemm_fp8(const GemmArgs& g, hipStream_t st) {
  if (g.K % kSlice2 != 0) return hipErrorInvalidValue;
  switch (g.y_dt) {
    case SQ_DT_F32: return launch_fp8_typed<SQ_DT_F32>(g, st);
    case SQ_DT_F16: return launch_fp8_typed<SQ_DT_F16>(g, st);
    case SQ_DT_BF16: return launch_fp8_typed<SQ_DT_BF16>(g, st);
    default: return hipErrorInvalidValue;
  }
}

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
