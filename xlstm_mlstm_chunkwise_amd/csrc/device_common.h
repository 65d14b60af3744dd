// Device helpers shared by the gfx950 mLSTM kernels: operand fragments for
// the 16x16 matrix-core tiles, dtype conversion, gate math and block scans.
//
// Matrix-core fragment convention (v_mfma_f32_16x16x32_f16 and, for float32
// inputs, eight v_mfma_f32_16x16x4_f32 steps): a fragment is the eight
// contraction-axis values one lane contributes to a 16 x 16 x 32 product.
// Lane l works on row / column (l % 16) of its operand and on contraction
// slots 8 * (l / 16) + e, e = 0..7.  Which contraction index sits in which
// slot is free as long as the A and B fragments of one product agree; the
// kernels use that freedom to feed accumulator tiles straight back in as
// operands.  The 16 x 16 float accumulator holds, in lane l register r, the
// element (row 4 * (l / 16) + r, column l % 16).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mlstm {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 storage type (raw bits) for inputs and outputs.
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even float -> bf16 (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7f800000u) == 0x7f800000u) return static_cast<uint16_t>((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// log(sigmoid(x)) without overflow: min(x, 0) - log1p(exp(-|x|)).
__device__ __forceinline__ float log_sigmoid(float x) {
  return fminf(x, 0.0f) - log1pf(expf(-fabsf(x)));
}

// ---------------------------------------------------------------------------
// Operand traits.  TIn is the storage type of Q, K, V.

template <typename TIn>
struct Ops;

// bf16 inputs: fp16 matrix-core operands (bf16 -> fp16 is exact for
// magnitudes in [2^-14, 65504]).
template <>
struct Ops<bf16_t> {
  typedef half8_t frag;
  typedef _Float16 lds_t;  // element type of staged input tiles
  static constexpr bool kSplitCapable = true;

  __device__ static __forceinline__ float4_t mma(const frag& a, const frag& b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ frag round(const float (&x)[8]) {
    frag f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = static_cast<_Float16>(x[e]);
    return f;
  }
  // x ~= hi + lo with hi = fp16(x), lo = fp16(x - hi).
  __device__ static __forceinline__ void split(const float (&x)[8], frag& hi, frag& lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      _Float16 h = static_cast<_Float16>(x[e]);
      hi[e] = h;
      lo[e] = static_cast<_Float16>(x[e] - static_cast<float>(h));
    }
  }
  __device__ static __forceinline__ lds_t to_lds(float x) { return static_cast<_Float16>(x); }
  // Store 8 floats as operand elements at p[0..7] (16-byte aligned).
  __device__ static __forceinline__ void store8(lds_t* p, const float (&x)[8]) {
    *reinterpret_cast<half8_t*>(p) = round(x);
  }
  // Load 8 consecutive inputs (16 bytes) and widen to float.
  __device__ static __forceinline__ void load8(const bf16_t* p, float (&x)[8]) {
    uint4 u = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(w[e] << 16);
      x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  }
  // Read a fragment of 8 staged elements at p[0..7] (16-byte aligned).
  __device__ static __forceinline__ frag lds_frag(const lds_t* p) {
    return *reinterpret_cast<const half8_t*>(p);
  }
  // Fragment from two runs of 4 staged elements (8-byte aligned each).
  __device__ static __forceinline__ frag lds_frag2(const lds_t* p0, const lds_t* p1) {
    typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
    half4_t a = *reinterpret_cast<const half4_t*>(p0);
    half4_t b = *reinterpret_cast<const half4_t*>(p1);
    frag f;
    f[0] = a[0]; f[1] = a[1]; f[2] = a[2]; f[3] = a[3];
    f[4] = b[0]; f[5] = b[1]; f[6] = b[2]; f[7] = b[3];
    return f;
  }
};

// float32 inputs: fp32 matrix-core operands, exact products.
struct f32frag {
  float v[8];
};

template <>
struct Ops<float> {
  typedef f32frag frag;
  typedef float lds_t;
  static constexpr bool kSplitCapable = false;

  __device__ static __forceinline__ float4_t mma(const frag& a, const frag& b, float4_t c) {
#pragma unroll
    for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], c, 0, 0, 0);
    return c;
  }
  __device__ static __forceinline__ frag round(const float (&x)[8]) {
    frag f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f.v[e] = x[e];
    return f;
  }
  __device__ static __forceinline__ void split(const float (&x)[8], frag& hi, frag& lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      hi.v[e] = x[e];
      lo.v[e] = 0.0f;
    }
  }
  __device__ static __forceinline__ lds_t to_lds(float x) { return x; }
  __device__ static __forceinline__ void store8(lds_t* p, const float (&x)[8]) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
  }
  __device__ static __forceinline__ void load8(const float* p, float (&x)[8]) {
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
  __device__ static __forceinline__ frag lds_frag(const lds_t* p) {
    frag f;
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
    return f;
  }
  __device__ static __forceinline__ frag lds_frag2(const lds_t* p0, const lds_t* p1) {
    frag f;
    float4 a = *reinterpret_cast<const float4*>(p0);
    float4 b = *reinterpret_cast<const float4*>(p1);
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
    return f;
  }
};

// acc += A . B with A computed in float (x); SPLIT carries A as hi + lo.
template <typename TIn, bool SPLIT>
__device__ __forceinline__ float4_t mma_computed_a(const float (&x)[8], const typename Ops<TIn>::frag& b,
                                                   float4_t acc) {
  typedef Ops<TIn> O;
  if constexpr (SPLIT && O::kSplitCapable) {
    typename O::frag hi, lo;
    O::split(x, hi, lo);
    acc = O::mma(hi, b, acc);
    acc = O::mma(lo, b, acc);
  } else {
    acc = O::mma(O::round(x), b, acc);
  }
  return acc;
}

// acc += A . B with B computed in float (x).
template <typename TIn, bool SPLIT>
__device__ __forceinline__ float4_t mma_computed_b(const typename Ops<TIn>::frag& a, const float (&x)[8],
                                                   float4_t acc) {
  typedef Ops<TIn> O;
  if constexpr (SPLIT && O::kSplitCapable) {
    typename O::frag hi, lo;
    O::split(x, hi, lo);
    acc = O::mma(a, hi, acc);
    acc = O::mma(a, lo, acc);
  } else {
    acc = O::mma(a, O::round(x), acc);
  }
  return acc;
}

// ---------------------------------------------------------------------------
// Block-wide inclusive scans over up to 4 * blockDim.x elements held 4 per
// thread (thread t holds positions 4t .. 4t+3).  NW = number of waves.

template <bool IS_MAX>
__device__ __forceinline__ float scan_op(float a, float b) {
  return IS_MAX ? fmaxf(a, b) : a + b;
}

// In-place inclusive scan of v[0..3] across the block.  `wave_tot` is LDS
// scratch of at least NW floats.  Contains __syncthreads().
template <bool IS_MAX, int NW>
__device__ __forceinline__ void block_scan4(float (&v)[4], float* wave_tot) {
  const float ident = IS_MAX ? -INFINITY : 0.0f;
  v[1] = scan_op<IS_MAX>(v[0], v[1]);
  v[2] = scan_op<IS_MAX>(v[1], v[2]);
  v[3] = scan_op<IS_MAX>(v[2], v[3]);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  float x = v[3];
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    float y = __shfl_up(x, off, 64);
    if (lane >= off) x = scan_op<IS_MAX>(y, x);
  }
  // x: inclusive over the wave's thread totals; exclusive = shift by one lane.
  float excl = __shfl_up(x, 1, 64);
  if (lane == 0) excl = ident;
  if (lane == 63) wave_tot[wave] = x;
  __syncthreads();
  float off_w = ident;
  for (int w = 0; w < wave; ++w) off_w = scan_op<IS_MAX>(off_w, wave_tot[w]);
  const float pre = scan_op<IS_MAX>(off_w, excl);
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = scan_op<IS_MAX>(pre, v[e]);
  __syncthreads();
}

// Block-wide reduction (max or sum) of one value per thread; result
// broadcast to all threads.  `scratch` holds >= NW floats.  Contains
// __syncthreads().
template <bool IS_MAX, int NW>
__device__ __forceinline__ float block_reduce(float x, float* scratch) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = scan_op<IS_MAX>(x, __shfl_xor(x, off, 64));
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = x;
  __syncthreads();
  float r = scratch[0];
  for (int w = 1; w < NW; ++w) r = scan_op<IS_MAX>(r, scratch[w]);
  __syncthreads();
  return r;
}

}  // namespace mlstm
