// Device helpers shared by the row kernels and the GEMM epilogues (gfx950, wave64).
//
// The library's numerical contract gives every binary32 operation its own
// round-to-nearest-even rounding: no multiply-add is contracted (the pragma
// below, also -ffp-contract=off on the command line), and division and square
// root are the IEEE-correct ones (the HIP default,
// -fhip-fp32-correctly-rounded-divide-sqrt). HIP's __fsqrt_rn is NOT used: it
// maps to the approximate hardware square root unless the ocml rounded
// operations are enabled.
#pragma once
#pragma clang fp contract(off)

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <cstdint>

namespace sq {

constexpr int kWave = 64;

// Correctly rounded binary32 operations (see the header comment).
__device__ __forceinline__ float add_rn(float a, float b) { return a + b; }
__device__ __forceinline__ float sub_rn(float a, float b) { return a - b; }
__device__ __forceinline__ float mul_rn(float a, float b) { return a * b; }
__device__ __forceinline__ float div_rn(float a, float b) { return a / b; }
__device__ __forceinline__ float sqrt_rn(float a) { return __builtin_sqrtf(a); }

// Make a register value opaque to the optimiser (no instruction emitted): a
// later pass over the same data then recomputes what it needs instead of the
// compiler keeping an earlier pass's intermediates alive, which would blow
// the register budget of a row held in registers.
__device__ __forceinline__ void opaque(float& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void opaque(uint4& v) { asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w)); }
__device__ __forceinline__ void memory_opaque() { asm volatile("" ::: "memory"); }

// ----------------------------------------------------------------------------- storage types
struct f32_t {};
struct f16_t {};
struct bf16_t {};

template <typename T> struct Storage;
template <> struct Storage<f32_t> { static constexpr int kBytes = 4; };
template <> struct Storage<f16_t> { static constexpr int kBytes = 2; };
template <> struct Storage<bf16_t> { static constexpr int kBytes = 2; };

__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits16) {
  return __half2float(__ushort_as_half(static_cast<unsigned short>(bits16)));
}

// Raw storage of 8 consecutive elements (one 16-byte load; two for binary32).
template <typename T> struct Raw8 { uint4 a; };
template <> struct Raw8<f32_t> { uint4 a, b; };

// Rows are streamed once, so the loads are non-temporal (they do not displace
// reused data from the caches).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
template <typename T> __device__ __forceinline__ void raw_load(const void* p, Raw8<T>& r) {
  r.a = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
}
template <> __device__ __forceinline__ void raw_load<f32_t>(const void* p, Raw8<f32_t>& r) {
  r.a = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
  r.b = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p) + 1));
}

// Rows through buffer resources: one resource per row (its base and size are
// workgroup-uniform, so they live in scalar registers and cost no vector
// instructions per row), and each thread's byte offsets within a row stay the
// same for every row. Offsets at or past `bytes` read zeros and drop writes.
constexpr int kBufNonTemporal = 2;           // buffer cache policy: streamed once
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}
template <typename T> __device__ __forceinline__ void raw_load_buf(__amdgpu_buffer_rsrc_t r, uint32_t off, Raw8<T>& v) {
  v.a = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kBufNonTemporal));
}
template <>
__device__ __forceinline__ void raw_load_buf<f32_t>(__amdgpu_buffer_rsrc_t r, uint32_t off, Raw8<f32_t>& v) {
  v.a = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kBufNonTemporal));
  v.b = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, kBufNonTemporal));
}
// 8 int8 codes (two packed words) at byte offset off, non-temporal: the codes
// are written once and read by a later kernel.
__device__ __forceinline__ void store_codes8_buf(__amdgpu_buffer_rsrc_t r, uint32_t off, uint2 w) {
  __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{w.x, w.y}, r, off, 0, kBufNonTemporal);
}
// 8 binary32 values (gamma, beta) at byte offset off, cached normally.
__device__ __forceinline__ void load8_f32_buf(__amdgpu_buffer_rsrc_t r, uint32_t off, float v[8]) {
  const u32x4_t a = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  const u32x4_t b = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 0);
  v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y); v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
  v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y); v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
}

// Widen 8 stored elements exactly to binary32.
template <typename T> __device__ __forceinline__ void widen8(const Raw8<T>& r, float v[8]);

template <> __device__ __forceinline__ void widen8<f32_t>(const Raw8<f32_t>& r, float v[8]) {
  v[0] = __uint_as_float(r.a.x); v[1] = __uint_as_float(r.a.y); v[2] = __uint_as_float(r.a.z);
  v[3] = __uint_as_float(r.a.w); v[4] = __uint_as_float(r.b.x); v[5] = __uint_as_float(r.b.y);
  v[6] = __uint_as_float(r.b.z); v[7] = __uint_as_float(r.b.w);
}

template <> __device__ __forceinline__ void widen8<f16_t>(const Raw8<f16_t>& r, float v[8]) {
  const uint32_t w[4] = {r.a.x, r.a.y, r.a.z, r.a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = f16_bits_to_f32(w[i] & 0xffffu);
    v[2 * i + 1] = f16_bits_to_f32(w[i] >> 16);
  }
}

template <> __device__ __forceinline__ void widen8<bf16_t>(const Raw8<bf16_t>& r, float v[8]) {
  const uint32_t w[4] = {r.a.x, r.a.y, r.a.z, r.a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// Load 8 consecutive elements (p is 16-byte aligned) and widen them exactly to binary32.
template <typename T> __device__ __forceinline__ void load8(const void* p, float v[8]) {
  Raw8<T> r;
  raw_load<T>(p, r);
  widen8<T>(r, v);
}

// 8 binary32 values from a 16-byte-aligned fp32 vector (gamma, beta, s).
__device__ __forceinline__ void load8_f32(const float* p, float v[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// ----------------------------------------------------------------------------- output conversion
// binary32 -> bfloat16 bits, round half to even (finite values).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t f32_to_f16_rne(float f) {
  return static_cast<uint32_t>(__half_as_ushort(__float2half_rn(f)));
}

// ----------------------------------------------------------------------------- reductions
// Wave reductions by DPP lane moves (no LDS round trips): inside each 16-lane
// row, exchange with lane ^ 1, ^ 2, then the mirrored lane of the half row and
// of the row; every step combines two equal-sized partial results in an order
// that is the same on both lanes, so all 16 lanes end with identical bits. The
// four row results are then combined in a fixed order from uniform values.
// (Every lane's source exists for these patterns, so no lane keeps an old
// value: the move needs no initialised destination.)
template <int CTRL>
__device__ __forceinline__ int dpp_move(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ double dpp_move(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const int lo = dpp_move<CTRL>(static_cast<int>(u & 0xffffffffu));
  const int hi = dpp_move<CTRL>(static_cast<int>(u >> 32));
  return __builtin_bit_cast(double, (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) |
                                        static_cast<uint32_t>(lo));
}
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(dpp_move<CTRL>(__float_as_int(v)));
}
__device__ __forceinline__ double read_lane(double v, int lane) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const int lo = __builtin_amdgcn_readlane(static_cast<int>(u & 0xffffffffu), lane);
  const int hi = __builtin_amdgcn_readlane(static_cast<int>(u >> 32), lane);
  return __builtin_bit_cast(double, (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) |
                                        static_cast<uint32_t>(lo));
}
__device__ __forceinline__ float read_lane(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

constexpr int kDppXor1 = 0xB1;           // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;           // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;    // row_half_mirror
constexpr int kDppMirror = 0x140;        // row_mirror

__device__ __forceinline__ double wave_sum(double v) {
  v += dpp_move<kDppXor1>(v);
  v += dpp_move<kDppXor2>(v);
  v += dpp_move<kDppHalfMirror>(v);
  v += dpp_move<kDppMirror>(v);
  return (read_lane(v, 0) + read_lane(v, 16)) + (read_lane(v, 32) + read_lane(v, 48));
}

// Max over a wave of non-negative binary32 values, taken on their bit patterns
// (for v >= 0 the IEEE order is the integer order), so each DPP step is a
// single v_max_i32 with a DPP source and the last step runs on scalar units.
__device__ __forceinline__ float wave_max_nonneg(float v) {
  int u = __float_as_int(v);
  u = max(u, dpp_move<kDppXor1>(u));
  u = max(u, dpp_move<kDppXor2>(u));
  u = max(u, dpp_move<kDppHalfMirror>(u));
  u = max(u, dpp_move<kDppMirror>(u));
  return __int_as_float(max(max(__builtin_amdgcn_readlane(u, 0), __builtin_amdgcn_readlane(u, 16)),
                            max(__builtin_amdgcn_readlane(u, 32), __builtin_amdgcn_readlane(u, 48))));
}

// Workgroup reductions with one barrier each: wave results go to LDS, and
// every thread combines them in a fixed order (deterministic run to run).
// Successive reductions must alternate between two buffers (RedRing): a
// buffer is written again only two reductions later, after a barrier that
// every thread reaches only once it has read the buffer's previous contents.
template <int THREADS>
struct RedRing {
  double buf[2][2 * (THREADS / kWave)];                  // room for two values per wave
  __device__ __forceinline__ double* at(int k) { return buf[k & 1]; }
};

template <int THREADS>
__device__ __forceinline__ double block_sum(double v, double* red) {
  constexpr int kWaves = THREADS / kWave;
  v = wave_sum(v);
  if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) t += red[i];
  return t;
}

// Two sums with one barrier (same order as block_sum for each).
template <int THREADS>
__device__ __forceinline__ void block_sum2(double& a, double& b, double* red) {
  constexpr int kWaves = THREADS / kWave;
  a = wave_sum(a);
  b = wave_sum(b);
  if (threadIdx.x % kWave == 0) {
    red[threadIdx.x / kWave] = a;
    red[kWaves + threadIdx.x / kWave] = b;
  }
  __syncthreads();
  double ta = 0.0, tb = 0.0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    ta += red[i];
    tb += red[kWaves + i];
  }
  a = ta;
  b = tb;
}

template <int THREADS>
__device__ __forceinline__ float block_max(float v, float* red) {   // v >= 0
  constexpr int kWaves = THREADS / kWave;
  v = wave_max_nonneg(v);
  if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = v;
  __syncthreads();
  const int* r = reinterpret_cast<const int*>(red);
  int t = r[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) t = max(t, r[i]);
  return __int_as_float(t);
}

// ----------------------------------------------------------------------------- INT8 codes
// Step of a row: fl32(absmax / 127), as fl32(fl64(absmax * fl64(1/127))).
// The binary64 value is within 2^-51 relative of q = absmax / 127, while q
// lies at least 2^-34 relative from every binary32 rounding boundary m near
// it: m is an odd multiple of half a binary32 spacing h of q's binade, and
// absmax, whose binade is 2^6 or 2^7 times higher (or, for a subnormal q, a
// multiple of the same fixed spacing), is an even multiple of h, so
// absmax - 127 m is a nonzero multiple of h and |q - m| >= h / 127. Both
// therefore round to the same binary32 value.
__device__ __forceinline__ float int8_step(float amax) {
  return static_cast<float>(static_cast<double>(amax) * (1.0 / 127.0));
}

// Per-row quantiser: code = clip(rne(fl32(y / step)), -127, 127).
//
// The quotient fl32(y / step) is needed only to decide which side of a
// half-integer it falls on. With r = v_rcp_f32(step), within one ulp (2^-23
// relative) of 1 / step for steps in [2^-100, 2^126] (inputs and results
// normal), the exact product P = y * r differs from the exact quotient Q by at
// most |Q| 2^-23, and fl32(Q) from Q by at most |Q| 2^-24, so for |Q| <= 128
// fl32(Q) lies within 1.5 * 2^-16 of P: rne(P) = rne(fl32(Q)) whenever P lies
// farther than that from every half-integer.
// One FMA gives s = fl(P + 1.5 * 2^23), which is 1.5 * 2^23 + rne(P) for
// |P| < 2^22 (the binary32 spacing there is 1, ties to even, and 1.5 * 2^23
// is even), so the low byte of s's bits is rne(P) in two's complement; a
// second FMA gives the residual d = fl(P - rne(P)) (one rounding of a value
// below 1/2, within 2^-25). Elements with |d| >= 1/2 - 2^-15 (P within about
// 2^-15 of a half-integer) take the IEEE division, and so do all elements for
// steps outside [2^-100, 2^126] (where 1/step would leave the normal range;
// only a step given for a whole tensor can exceed 2^126).
struct Quantizer {
  static constexpr float kMagic = 12582912.0f;         // 1.5 * 2^23
  float step, rcp;
  bool zero, exact_only;
  __device__ __forceinline__ explicit Quantizer(float st) : step(st) {
    zero = !(st > 0.0f);
    exact_only = !(st >= 0x1p-100f && st <= 0x1p126f);
    rcp = __builtin_amdgcn_rcpf(st);                     // v_rcp_f32: within one ulp of 1 / st
  }
  // Codes of 8 values, packed little-endian into two 32-bit words. With the
  // row's own step |P| <= amax * r < 127.5, so rne(P) needs no
  // clamp; CLIP (a step given for a whole tensor, which values may exceed)
  // clamps s to 1.5 * 2^23 +- 127. For |P| >= 2^22 s is no longer
  // 1.5 * 2^23 + rne(P), but it stays on P's side of that range, so the clamp
  // still gives +-127 (a product that overflows fails the residual test and
  // divides). The exact path always clamps (a subnormal step may push the
  // quotient past 127). One comparison covers all 8 elements: the largest
  // |d|. (NaN and Inf inputs are outside the contract; such elements get
  // some code.)
  template <bool CLIP = false>
  __device__ __forceinline__ uint2 codes8(const float y[8]) const {
    if (zero) return make_uint2(0u, 0u);                 // workgroup-uniform
    float m[8], d[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      m[i] = __builtin_fmaf(y[i], rcp, kMagic);
      d[i] = __builtin_fmaf(y[i], rcp, kMagic - m[i]);  // kMagic - m[i] = -rne(P), exact
    }
    float dm = fabsf(d[0]);
#pragma unroll
    for (int i = 1; i < 8; ++i) dm = fmaxf(dm, fabsf(d[i]));
    if (exact_only || !(dm < 0.499969482421875f)) {     // 0.5 - 2^-15
#pragma unroll
      for (int i = 0; i < 8; ++i) m[i] = kMagic + fminf(fmaxf(rintf(div_rn(y[i], step)), -127.0f), 127.0f);
    } else if constexpr (CLIP) {
#pragma unroll
      for (int i = 0; i < 8; ++i) m[i] = fminf(fmaxf(m[i], kMagic - 127.0f), kMagic + 127.0f);
    }
    uint32_t c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = __float_as_uint(m[i]);
    // low bytes: perm(hi, lo, sel) picks bytes of {hi:lo}; 0x0c gives 0x00
    const uint32_t w0 = __builtin_amdgcn_perm(c[1], c[0], 0x0c0c0400u) | __builtin_amdgcn_perm(c[3], c[2], 0x04000c0cu);
    const uint32_t w1 = __builtin_amdgcn_perm(c[5], c[4], 0x0c0c0400u) | __builtin_amdgcn_perm(c[7], c[6], 0x04000c0cu);
    return make_uint2(w0, w1);
  }
};

// Per-row FP8 step: fl32(absmax / 448), 448 being OCP E4M3's largest finite value.
__device__ __forceinline__ float fp8_step(float amax) { return div_rn(amax, 448.0f); }

// Per-row FP8 quantiser: code = E4M3(fl32(y / step)), round half to even
// (v_cvt_pk_fp8_f32 rounds that way; gfx950 converts to OCP E4M3). Here
// t = fl32(y * fl32(1 / step)) stands in for the quotient q: with
// |t| in [2^e, 2^(e+1)), |t - q| <= |q| 2^-23 (1 + 2^-25) is below 2.0001 ulps
// of t, and below one ulp of t when q < 2^e, so q lies strictly between the
// binary32 values 4 bit steps below and above t (the step below 2^e is half
// as wide). E4M3 rounding is monotone: when those two neighbours get the same
// code, q gets it too; otherwise (a midpoint lies between them, in E4M3's
// normal or subnormal range alike) the codes come from exact quotients. The
// step below saturates at +0 (a zero y keeps its zero code); below -0 it
// wraps to a NaN pattern, which only sends those 8 values to the exact path.
// With the row's own step |t| stays within 448 * (1 + 2^-23), below the 464
// midpoint past which E4M3 has only NaN. CLIP (a step given for a whole
// tensor, which values may exceed) saturates t, and the exact quotients, to
// [-448, 448] first: sat(q) then lies between the neighbours of sat(t) (both
// sides of 448 are in one binade, and beyond 448 both neighbours take 448's
// code), so the neighbour test still decides.
struct QuantizerFp8 {
  float step, rcp;
  bool zero, exact_only;
  __device__ __forceinline__ explicit QuantizerFp8(float st) : step(st) {
    zero = !(st > 0.0f);
    exact_only = st < 0x1p-100f;
    rcp = zero ? 0.0f : div_rn(1.0f, st);
  }
  __device__ __forceinline__ static uint2 pack8(const float t[8]) {
    int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(t[0], t[1], 0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(t[2], t[3], w0, true);
    int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(t[4], t[5], 0, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(t[6], t[7], w1, true);
    return make_uint2(static_cast<uint32_t>(w0), static_cast<uint32_t>(w1));
  }
  __device__ __forceinline__ static float sat(float v) { return fminf(fmaxf(v, -448.0f), 448.0f); }
  template <bool CLIP = false>
  __device__ __forceinline__ uint2 codes8(const float y[8]) const {
    if (zero) return make_uint2(0u, 0u);                 // workgroup-uniform
    float lo[8], hi[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float t = mul_rn(y[i], rcp);
      const uint32_t u = __float_as_uint(CLIP ? sat(t) : t);
      lo[i] = __uint_as_float(__builtin_elementwise_sub_sat(u, 4u));
      hi[i] = __uint_as_float(u + 4u);
    }
    const uint2 a = pack8(lo), b = pack8(hi);
    if (!exact_only && a.x == b.x && a.y == b.y) return a;
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = CLIP ? sat(div_rn(y[i], step)) : div_rn(y[i], step);
    return pack8(t);
  }
};

// Max over non-negative binary32 values through their bit patterns (IEEE order
// equals unsigned order there), order-independent and exact.
__device__ __forceinline__ void atomic_max_nonneg(float* addr, float v) {
  atomicMax(reinterpret_cast<unsigned int*>(addr), __float_as_uint(v));
}

}  // namespace sq
