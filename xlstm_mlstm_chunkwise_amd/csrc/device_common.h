// Device helpers shared by the gfx950 mLSTM kernels: operand fragments for
// the 16x16 matrix-core tiles, dtype conversion, gate math and block scans.
//
// Matrix-core fragment convention (v_mfma_f32_16x16x32_bf16 and, for float32
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

// bf16 inputs: bf16 matrix-core operands.  Q, K, V enter unchanged (every
// bf16 value, of any magnitude, is exact); an operand computed in float32 is
// rounded to bf16, or carried as a bf16 hi + lo pair (about 16 significant
// bits).
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <>
struct Ops<bf16_t> {
  typedef bf16x8_t frag;
  typedef __bf16 lds_t;  // element type of staged input tiles
  static constexpr bool kSplitCapable = true;

  __device__ static __forceinline__ float4_t mma(const frag& a, const frag& b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ frag round(const float (&x)[8]) {
    frag f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = static_cast<__bf16>(x[e]);
    return f;
  }
  // x ~= hi + lo with hi = bf16(x), lo = bf16(x - hi).
  __device__ static __forceinline__ void split(const float (&x)[8], frag& hi, frag& lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const __bf16 h = static_cast<__bf16>(x[e]);
      hi[e] = h;
      lo[e] = static_cast<__bf16>(x[e] - static_cast<float>(h));
    }
  }
  __device__ static __forceinline__ lds_t to_lds(float x) { return static_cast<__bf16>(x); }
  // Store 8 floats as operand elements at p[0..7] (16-byte aligned).
  __device__ static __forceinline__ void store8(lds_t* p, const float (&x)[8]) {
    *reinterpret_cast<bf16x8_t*>(p) = round(x);
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
    return *reinterpret_cast<const bf16x8_t*>(p);
  }
  // Fragment from two runs of 4 staged elements (8-byte aligned each).
  __device__ static __forceinline__ frag lds_frag2(const lds_t* p0, const lds_t* p1) {
    const bf16x4_t a = *reinterpret_cast<const bf16x4_t*>(p0);
    const bf16x4_t b = *reinterpret_cast<const bf16x4_t*>(p1);
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


// ---------------------------------------------------------------------------
// 32x32x16 fp16 matrix-core tiles (v_mfma_f32_32x32x16_f16).
// A fragment: lane l holds A[row l % 32][k 8 * (l / 32) + e], e = 0..7.
// B fragment: lane l holds B[k 8 * (l / 32) + e][col l % 32].
// Accumulator: lane l register r holds D[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32].

typedef float float16_t __attribute__((ext_vector_type(16)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float16_t mma32(const half8_t& a, const half8_t& b, float16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Transposing LDS read (ds_read_b64_tr_b16): within each group of 16 lanes,
// lane i receives element e = 0..3 from address a_{i/4 + 4e} + (i % 4),
// where a_j is the address supplied by lane j of the group.
typedef short short4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ half4_t lds_read_tr16(const _Float16* p) {
  const short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)(p));
  return __builtin_bit_cast(half4_t, v);
}

// Fragment whose contraction axis runs down the rows of a row-major LDS
// matrix X (row stride ld elements): lane l gets X[k0 + 8 * (l / 32) + e][c0 + l % 32],
// e = 0..7.  Serves as a B fragment (rows = k, columns = n) and as an A
// fragment of the transposed matrix (columns of X = rows of A).
__device__ __forceinline__ half8_t frag_tr(const _Float16* X, int ld, int k0, int c0, int lane) {
  const int grp = lane >> 4, j = lane & 15;
  const _Float16* base = X + (k0 + 8 * (grp >> 1) + (j >> 2)) * ld + c0 + 16 * (grp & 1) + 4 * (j & 3);
  const half4_t lo = lds_read_tr16(base);
  const half4_t hi = lds_read_tr16(base + 4 * ld);
  half8_t f;
  f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
  f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
  return f;
}

// Fragment whose contraction axis runs along a row of a row-major LDS matrix:
// lane l gets X[r0 + l % 32][k0 + 8 * (l / 32) + e] (one 16-byte read).
__device__ __forceinline__ half8_t frag_row(const _Float16* X, int ld, int r0, int k0, int lane) {
  return *reinterpret_cast<const half8_t*>(X + (r0 + (lane & 31)) * ld + k0 + 8 * (lane >> 5));
}

// bf16 x 8 (16 bytes) -> fp16 x 8.
__device__ __forceinline__ half8_t bf16x8_to_f16x8(uint4 u) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  half8_t f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = static_cast<_Float16>(__uint_as_float(w[e] << 16));
    f[2 * e + 1] = static_cast<_Float16>(__uint_as_float(w[e] & 0xffff0000u));
  }
  return f;
}

// ---------------------------------------------------------------------------
// Packed chunk-state layout shared by the wide states and intra-chunk kernels.
// One state (DK x DV) is stored as (DK/16) x (DV/32) fragments of a 16-row k
// step and a 32-column block; each fragment is a hi plane then a lo plane of
// 64 lanes x 8 bf16 values (2 x 1 KiB).  Lane l holds column 32*nb + l % 32;
// slot e holds row 16*kk + (e < 4 ? 4*(l/32) + e : 8 + 4*(l/32) + e - 4), the
// row order of a 32x32 accumulator half.  hi + lo reproduces the float32
// state to about 16 significant bits.
__device__ __forceinline__ size_t pack_frag_offset(int kk, int nb, int plane, int DV) {
  return ((size_t)(kk * (DV / 32) + nb) * 2 + plane) * 512;
}

// 4 bf16 (8 bytes) -> 4 fp16.
__device__ __forceinline__ half4_t bf16x4_to_f16x4(uint2 u) {
  half4_t f;
  f[0] = static_cast<_Float16>(__uint_as_float(u.x << 16));
  f[1] = static_cast<_Float16>(__uint_as_float(u.x & 0xffff0000u));
  f[2] = static_cast<_Float16>(__uint_as_float(u.y << 16));
  f[3] = static_cast<_Float16>(__uint_as_float(u.y & 0xffff0000u));
  return f;
}

// ---------------------------------------------------------------------------
// bf16 matrix-core operands (wide kernels).  Inputs Q, K, V feed the bf16
// MFMAs unchanged; a value computed in float32 is carried as a bf16 hi + lo
// pair (hi = RNE(x), lo = RNE(x - hi)), about 16 significant bits.

__device__ __forceinline__ float16_t mma32b(const bf16x8_t& a, const bf16x8_t& b, float16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float4_t mma16b(const bf16x8_t& a, const bf16x8_t& b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Two floats -> packed bf16 hi and lo words (low half = first value).
__device__ __forceinline__ void split_bf16x2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  bf16x2_t h;
  h[0] = static_cast<__bf16>(x0);
  h[1] = static_cast<__bf16>(x1);
  hi = __builtin_bit_cast(uint32_t, h);
  const float h0 = __uint_as_float(hi << 16), h1 = __uint_as_float(hi & 0xffff0000u);
  bf16x2_t l;
  l[0] = static_cast<__bf16>(x0 - h0);
  l[1] = static_cast<__bf16>(x1 - h1);
  lo = __builtin_bit_cast(uint32_t, l);
}

__device__ __forceinline__ uint32_t round_bf16x2(float x0, float x1) {
  bf16x2_t h;
  h[0] = static_cast<__bf16>(x0);
  h[1] = static_cast<__bf16>(x1);
  return __builtin_bit_cast(uint32_t, h);
}

// 16-bit fragment helpers on raw storage (bit patterns only).
__device__ __forceinline__ uint4 frag_tr_u(const uint16_t* X, int ld, int k0, int c0, int lane) {
  const int grp = lane >> 4, j = lane & 15;
  const uint16_t* base = X + (k0 + 8 * (grp >> 1) + (j >> 2)) * ld + c0 + 16 * (grp & 1) + 4 * (j & 3);
  const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)(base));
  const short4_t hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)(base + 4 * ld));
  const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
  return make_uint4(a.x, a.y, b.x, b.y);
}
__device__ __forceinline__ uint4 frag_row_u(const uint16_t* X, int ld, int r0, int k0, int lane) {
  return *reinterpret_cast<const uint4*>(X + (r0 + (lane & 31)) * ld + k0 + 8 * (lane >> 5));
}
__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

// Raw buffer access: a 128-bit resource (base address, byte extent, 32-bit
// data format for untyped loads) in scalar registers and a per-lane byte
// offset.  The hardware range check covers the lane offset and the
// instruction's immediate offset, not the scalar offset operand, so these
// helpers use no scalar offset where a row can lie past the data: a
// wave-uniform offset (a row block, a tile start) is folded into the resource
// by make_rsrc_at instead, which moves the base and shrinks the extent, and
// the steps inside a tile go in the lane offset.  Reads at or past the extent return
// zero and stores there are dropped.
typedef int v4i32_t __attribute__((ext_vector_type(4)));
typedef int v2i32_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// The bytes [off, extent) of the range at `base`, as a resource starting at
// base + off (empty when off >= extent).  off must be wave-uniform.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_at(const void* base, uint32_t extent, uint32_t off) {
  return make_rsrc(static_cast<const char*>(base) + off, off < extent ? extent - off : 0u);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, int voff) {
  const v4i32_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
  return make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
}

// The same with the non-temporal hint (aux 2), for data read once that should
// not displace lines other workgroups re-read from L2.
__device__ __forceinline__ uint4 buf_load16_nt(__amdgpu_buffer_rsrc_t r, int voff) {
  const v4i32_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 2);
  return make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
}
// A load with a scalar offset, for a resource every byte of which the
// kernel reads whole (a complete chunk state): soff + voff is in range by
// construction, so the unchecked scalar offset cannot reach past the data.
__device__ __forceinline__ uint4 buf_load16_whole(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const v4i32_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
}

__device__ __forceinline__ float unpack_state_elem_bf16(const uint16_t* P, int k, int v, int DV) {
  const int kk = k >> 4, kr = k & 15, nb = v >> 5, col = v & 31;
  const int h = (kr & 7) >> 2;
  const int e = (kr < 8 ? 0 : 4) + (kr & 3);
  const int lane = 32 * h + col;
  const float hi = bf16_to_f32(P[pack_frag_offset(kk, nb, 0, DV) + lane * 8 + e]);
  const float lo = bf16_to_f32(P[pack_frag_offset(kk, nb, 1, DV) + lane * 8 + e]);
  return hi + lo;
}

}  // namespace mlstm
