// One time step of the mLSTM recurrence for every head (decode), gfx950.
//
// The model configuration of "xLSTM: the NX-AI repository behind the extended
// LSTM architecture" (section "Exponential gating, matrix memory, and why the
// kernels decide everything") names a step kernel beside the chunkwise and
// sequence kernels: generation advances the matrix memory one token at a
// time.  Per head, from the state (C, n, m) entering the step, in the
// stabilised convention of the forward pass's final state, and the step's
// q, k, v and gate pre-activations, with lf = log sigmoid(f) and s the query
// scale:
//   exp gate:  m' = max(lf + m, i),  a = e^{lf + m - m'},  b = e^{i - m'}
//              C' = a C + b k v^T,   n' = a n + b k
//              h  = s C'^T q / (max(|s n' . q|, e^{-m'}) + eps)
//   sig gate:  C' = sigmoid(f) C + sigmoid(i) k v^T,   h = s C'^T q
//
// The step reads and writes the DHQK x DHV float32 state once and does two
// flops per element besides, so it is bound by memory.  One workgroup per
// (head, slice of C's columns): 128 columns and 512 threads where DHV is a
// multiple of 128, else 64 columns and 256 threads.  Thread (row group g,
// column quad c) streams the 16-byte pieces of rows g, g + 16, ... of its four
// columns (all its loads issued up front), applies the update, writes them
// back and accumulates s C'^T q; a reduction over the 16 row groups in LDS
// gives h.  The state is read and written with non-temporal accesses: in a
// model each layer's state is touched once per token, so between two steps of
// one layer the other layers' states have passed through the caches, and
// streaming them past the Infinity Cache measured about a quarter faster than
// ordinary accesses when the states exceed it.  Every workgroup of a head
// forms n' and m', which its normaliser needs; the first slice writes them.
//
// Quantised state (Q8): the "flash-xlstm-exp 0.1.0" page (section "Upgrade
// roadmap") lists an fp8/int8 memory state for long-context inference.  Here
// C is held as int8 codes with one float32 scale per block of 64 consecutive
// values of a row; a block x encodes as code = round-half-even(x * 127 / amax)
// with scale amax / 127 (all zeros when amax = 0).  The step decodes its
// pieces, updates them in float32, reads h from the updated values and
// encodes them again: the 16 threads that hold one block's 64 values (one DPP
// row of 16 lanes) find its amax with four DPP max steps, and 127 / amax
// comes from the reciprocal instruction (1 ulp).  In this mode each thread
// holds a run of DHQK/16 consecutive rows, so the scales, stored block-major
// (BH, DHV/64, DHQK), move in 16-byte pieces.  The state moves in 1 + 1/16
// bytes per value instead of 4.
#include "device_common.h"
#include "kernels.h"

namespace mlstm {
namespace {

constexpr int kStepGroups = 16;  // row groups per workgroup (float state)
constexpr int kQ8Groups = 32;    // row groups per workgroup (quantised state), at most
constexpr int kQ8Cols = 128;     // columns per workgroup (quantised state), at most

// Row groups of a workgroup: the quantised state keeps runs of at least four
// rows per thread (its scales move in 16-byte pieces).
template <int DK, bool Q8>
constexpr int step_groups() {
  return Q8 ? (DK / 4 < kQ8Groups ? DK / 4 : kQ8Groups) : kStepGroups;
}

typedef float step_f4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 load_stream(const float* a) {
  const step_f4_t x = __builtin_nontemporal_load(reinterpret_cast<const step_f4_t*>(a));
  return make_float4(x.x, x.y, x.z, x.w);
}

__device__ __forceinline__ void store_stream(float* a, float4 c) {
  const step_f4_t x = {c.x, c.y, c.z, c.w};
  __builtin_nontemporal_store(x, reinterpret_cast<step_f4_t*>(a));
}

// The code of x as the low byte of fma(x, inv, 1.5 * 2^23): for |x * inv| <
// 2^22 the sum lies where floats are spaced by one, so the single rounding of
// the fma is round-half-even of x * inv, and the low mantissa bits hold it in
// two's complement.  |x * inv| <= 127 (1 + 2^-21) for |x| <= amax, which
// rounds into [-127, 127].
__device__ __forceinline__ uint32_t encode_bits(float x, float inv) {
  return __float_as_uint(fmaf(x, inv, 12582912.0f));
}

// Low bytes of four words into one word (byte i from word i).
__device__ __forceinline__ uint32_t pack_low_bytes(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3) {
  const uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);
  const uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// DPP controls for the block maximum over the 16 lanes of a DPP row: swap
// within quads (0xB1: xor 1, 0x4E: xor 2), then mirror within half-rows
// (0x141) and within the row (0x140).

template <int DK, bool SIG, int COLS, bool Q8>
__global__ __launch_bounds__((COLS / 4 * step_groups<DK, Q8>())) void step_kernel(const StepParams p) {
  constexpr int RG = step_groups<DK, Q8>();         // row groups
  constexpr int THREADS = COLS / 4 * RG;            // COLS / 4 column quads x RG row groups
  constexpr int RPT = DK / RG;                      // rows per thread
  __shared__ float s_q[DK], s_k[DK];
  __shared__ float4 s_red[RG][COLS / 4];
  __shared__ float s_dot[THREADS / 64];

  const int DV = p.DV;
  const int NS = DV / COLS;
  const int bh = blockIdx.x / NS, slice = blockIdx.x % NS;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cq = tid % (COLS / 4), rg = tid / (COLS / 4);
  const int col = slice * COLS + 4 * cq;

  // gate factors of the step (every thread, from two scalars)
  const float lf = log_sigmoid(p.f_pre[bh]);
  const float ip = p.i_pre[bh];
  float a, b, m_new = 0.0f;
  if constexpr (SIG) {
    a = expf(lf);
    b = 1.0f / (1.0f + expf(-ip));
  } else {
    const float m_old = p.m_in ? p.m_in[bh] : 0.0f;
    m_new = fmaxf(lf + m_old, ip);
    a = expf(lf + m_old - m_new);
    b = expf(ip - m_new);
  }

  // this thread's pieces of the state go out first: they depend on nothing
  // else, and their latency then overlaps the staging of q and k
  const size_t cbase = (size_t)bh * DK * DV + col;
  // row of this thread's r-th piece: strided for the float state, a run of
  // RPT consecutive rows for the quantised one
  auto row_of = [&](int r) { return Q8 ? rg * RPT + r : rg + RG * r; };
  // scales of this thread's block, block-major: (BH, DV/64, DK)
  const size_t sbase = ((size_t)bh * (DV / 64) + col / 64) * DK + (size_t)rg * RPT;
  float4 cr[RPT];
  uint32_t cw[Q8 ? RPT : 1];
  float cs[Q8 ? RPT : 1];
  if constexpr (Q8) {
    static_assert(RPT % 4 == 0, "scales move in groups of four rows");
    if (p.Cq_in) {
#pragma unroll
      for (int r = 0; r < RPT; ++r)
        cw[r] = __builtin_nontemporal_load(
            reinterpret_cast<const uint32_t*>(p.Cq_in + cbase + (size_t)row_of(r) * DV));
#pragma unroll
      for (int r = 0; r < RPT; r += 4) {
        const float4 s4 = *reinterpret_cast<const float4*>(p.Cs_in + sbase + r);
        cs[r] = s4.x;
        cs[r + 1] = s4.y;
        cs[r + 2] = s4.z;
        cs[r + 3] = s4.w;
      }
    } else {
#pragma unroll
      for (int r = 0; r < RPT; ++r) {
        cw[r] = 0u;
        cs[r] = 0.0f;
      }
    }
  } else {
    if (p.C_in) {
#pragma unroll
      for (int r = 0; r < RPT; ++r) cr[r] = load_stream(p.C_in + cbase + (size_t)(rg + kStepGroups * r) * DV);
    } else {
#pragma unroll
      for (int r = 0; r < RPT; ++r) cr[r] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
  }

  // q (scaled) and k in LDS as float32; this thread's four values of v
  auto ld = [&](const void* x, size_t i) -> float {
    return p.qkv_bf16 ? bf16_to_f32(static_cast<const uint16_t*>(x)[i]) : static_cast<const float*>(x)[i];
  };
  for (int i = tid; i < DK; i += THREADS) {
    s_q[i] = p.scale * ld(p.q, (size_t)bh * DK + i);
    s_k[i] = ld(p.k, (size_t)bh * DK + i);
  }
  float4 v4;
  if (p.qkv_bf16) {
    const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p.v) + (size_t)bh * DV + col);
    v4 = make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                     __uint_as_float(u.y & 0xffff0000u));
  } else {
    v4 = *reinterpret_cast<const float4*>(static_cast<const float*>(p.v) + (size_t)bh * DV + col);
  }
  __syncthreads();

  // ---- the state update C' = a C + b k v^T, and s C'^T q for four columns
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if constexpr (Q8) {
    // in phases over the thread's rows, so that the block maxima of all rows
    // go through the DPP steps side by side
    float4 cn[RPT];
    float mx[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int row = row_of(r);
      const float bk = b * s_k[row], qv = s_q[row];
      // a (code * scale) + bk v with the code read as the unsigned byte
      // code + 128: (code + 128) (a scale) + (bk v - 128 a scale)
      const uint32_t u = cw[r] ^ 0x80808080u;
      const float as = a * cs[r], nb = -128.0f * as;
      float4 c;
      c.x = fmaf((float)(u & 0xffu), as, fmaf(bk, v4.x, nb));
      c.y = fmaf((float)((u >> 8) & 0xffu), as, fmaf(bk, v4.y, nb));
      c.z = fmaf((float)((u >> 16) & 0xffu), as, fmaf(bk, v4.z, nb));
      c.w = fmaf((float)(u >> 24), as, fmaf(bk, v4.w, nb));
      acc.x += c.x * qv;
      acc.y += c.y * qv;
      acc.z += c.z * qv;
      acc.w += c.w * qv;
      cn[r] = c;
      mx[r] = fmaxf(fmaxf(fabsf(c.x), fabsf(c.y)), fmaxf(fabsf(c.z), fabsf(c.w)));
    }
    // amax of each 64-value block over its 16 threads (one DPP row); the
    // values are >= 0, whose bit patterns order as unsigned integers
    uint32_t mb[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) mb[r] = __float_as_uint(mx[r]);
#pragma unroll
    for (int r = 0; r < RPT; ++r) mb[r] = max(mb[r], (uint32_t)__builtin_amdgcn_mov_dpp((int)mb[r], 0xB1, 0xF, 0xF, true));
#pragma unroll
    for (int r = 0; r < RPT; ++r) mb[r] = max(mb[r], (uint32_t)__builtin_amdgcn_mov_dpp((int)mb[r], 0x4E, 0xF, 0xF, true));
#pragma unroll
    for (int r = 0; r < RPT; ++r) mb[r] = max(mb[r], (uint32_t)__builtin_amdgcn_mov_dpp((int)mb[r], 0x141, 0xF, 0xF, true));
#pragma unroll
    for (int r = 0; r < RPT; ++r) mb[r] = max(mb[r], (uint32_t)__builtin_amdgcn_mov_dpp((int)mb[r], 0x140, 0xF, 0xF, true));
#pragma unroll
    for (int r = 0; r < RPT; ++r) mx[r] = __uint_as_float(mb[r]);
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const float m = mx[r];
      const float inv = m >= 1.17549435e-38f ? 127.0f * __builtin_amdgcn_rcpf(m) : (m > 0.0f ? 127.0f / m : 0.0f);
      const float4 c = cn[r];
      const uint32_t w = pack_low_bytes(encode_bits(c.x, inv), encode_bits(c.y, inv), encode_bits(c.z, inv),
                                        encode_bits(c.w, inv));
      __builtin_nontemporal_store(w, reinterpret_cast<uint32_t*>(p.Cq_out + cbase + (size_t)row_of(r) * DV));
    }
    if ((cq & 15) == 0) {
      constexpr float k127 = 1.0f / 127.0f;
#pragma unroll
      for (int r = 0; r < RPT; r += 4)
        *reinterpret_cast<float4*>(p.Cs_out + sbase + r) =
            make_float4(mx[r] * k127, mx[r + 1] * k127, mx[r + 2] * k127, mx[r + 3] * k127);
    }
  } else {
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int row = row_of(r);
      const float bk = b * s_k[row], qv = s_q[row];
      float4 c = cr[r];
      c.x = a * c.x + bk * v4.x;
      c.y = a * c.y + bk * v4.y;
      c.z = a * c.z + bk * v4.z;
      c.w = a * c.w + bk * v4.w;
      store_stream(p.C_out + cbase + (size_t)row * DV, c);
      acc.x += c.x * qv;
      acc.y += c.y * qv;
      acc.z += c.z * qv;
      acc.w += c.w * qv;
    }
  }
  s_red[rg][cq] = acc;

  // ---- normaliser s n' . q (exp gate), n' written by the first slice
  float den = 0.0f;
  if constexpr (!SIG) {
    float d = 0.0f;
    for (int i = tid; i < DK; i += THREADS) {
      const float n_new = a * (p.n_in ? p.n_in[(size_t)bh * DK + i] : 0.0f) + b * s_k[i];
      if (slice == 0 && p.n_out) p.n_out[(size_t)bh * DK + i] = n_new;
      d += n_new * s_q[i];
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) d += __shfl_xor(d, o, 64);
    if (lane == 0) s_dot[wave] = d;
  }
  __syncthreads();
  if constexpr (!SIG) {
#pragma unroll
    for (int w = 0; w < THREADS / 64; ++w) den += s_dot[w];
    if (slice == 0 && tid == 0 && p.m_out) p.m_out[bh] = m_new;
  }

  // ---- h for this slice's columns
  if (rg == 0) {
    float4 num = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      const float4 x = s_red[g][cq];
      num.x += x.x;
      num.y += x.y;
      num.z += x.z;
      num.w += x.w;
    }
    float inv = 1.0f;
    if constexpr (!SIG) inv = 1.0f / (fmaxf(fabsf(den), expf(-m_new)) + p.eps);
    const float hv[4] = {num.x * inv, num.y * inv, num.z * inv, num.w * inv};
    if (p.h_bf16) {
      uint16_t* H = static_cast<uint16_t*>(p.h) + (size_t)bh * DV + col;
      const uint2 u = make_uint2((uint32_t)f32_to_bf16(hv[0]) | ((uint32_t)f32_to_bf16(hv[1]) << 16),
                                 (uint32_t)f32_to_bf16(hv[2]) | ((uint32_t)f32_to_bf16(hv[3]) << 16));
      *reinterpret_cast<uint2*>(H) = u;
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(p.h) + (size_t)bh * DV + col) =
          make_float4(hv[0], hv[1], hv[2], hv[3]);
    }
  }
}

template <int DK, int COLS, bool Q8>
hipError_t launch_cols(const StepParams& p, bool sig, hipStream_t stream) {
  const dim3 grid((unsigned)((long long)p.BH * (p.DV / COLS)));
  const dim3 block(COLS / 4 * step_groups<DK, Q8>());
  if (sig) hipLaunchKernelGGL((step_kernel<DK, true, COLS, Q8>), grid, block, 0, stream, p);
  else hipLaunchKernelGGL((step_kernel<DK, false, COLS, Q8>), grid, block, 0, stream, p);
  return hipGetLastError();
}

template <int DK>
hipError_t launch_dk(const StepParams& p, bool sig, hipStream_t stream) {
  if (p.q8) {
    if (kQ8Cols == 128 && p.DV % 128 == 0) return launch_cols<DK, 128, true>(p, sig, stream);
    return launch_cols<DK, 64, true>(p, sig, stream);
  }
  return p.DV % 128 == 0 ? launch_cols<DK, 128, false>(p, sig, stream) : launch_cols<DK, 64, false>(p, sig, stream);
}

// Encoding / decoding of a whole float32 state (BH, DK, DV): one wave per
// 64-value block; block b of row r of head bh has its scale at
// ((bh * DV/64) + b) * DK + r.
__device__ __forceinline__ long long scale_index(long long blk, int DK, int NB) {
  const long long row = blk / NB;  // bh * DK + r
  return ((row / DK) * NB + blk % NB) * DK + row % DK;
}

__global__ __launch_bounds__(256) void q8_encode_kernel(const float* __restrict__ C, int8_t* __restrict__ Cq,
                                                        float* __restrict__ Cs, long long nblocks, int DK, int NB) {
  const long long blk = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (blk >= nblocks) return;
  const int lane = threadIdx.x & 63;
  const float x = C[blk * 64 + lane];
  float mx = fabsf(x);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  const float inv = mx > 0.0f ? 127.0f / mx : 0.0f;
  Cq[blk * 64 + lane] = (int8_t)(int)rintf(x * inv);
  if (lane == 0) Cs[scale_index(blk, DK, NB)] = mx / 127.0f;
}

__global__ __launch_bounds__(256) void q8_decode_kernel(const int8_t* __restrict__ Cq, const float* __restrict__ Cs,
                                                        float* __restrict__ C, long long nblocks, int DK, int NB) {
  const long long blk = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (blk >= nblocks) return;
  const int lane = threadIdx.x & 63;
  C[blk * 64 + lane] = (float)Cq[blk * 64 + lane] * Cs[scale_index(blk, DK, NB)];
}

}  // namespace

hipError_t launch_q8_encode(const float* C, int8_t* Cq, float* Cs, long long BH, int DK, int DV,
                            hipStream_t stream) {
  const long long nb = BH * DK * (DV / 64);
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL(q8_encode_kernel, dim3((unsigned)((nb + 3) / 4)), dim3(256), 0, stream, C, Cq, Cs, nb, DK,
                     DV / 64);
  return hipGetLastError();
}

hipError_t launch_q8_decode(const int8_t* Cq, const float* Cs, float* C, long long BH, int DK, int DV,
                            hipStream_t stream) {
  const long long nb = BH * DK * (DV / 64);
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL(q8_decode_kernel, dim3((unsigned)((nb + 3) / 4)), dim3(256), 0, stream, Cq, Cs, C, nb, DK,
                     DV / 64);
  return hipGetLastError();
}

hipError_t launch_step(const StepParams& p, bool sig, hipStream_t stream) {
  if (p.BH == 0) return hipSuccess;
  if (p.DV <= 0 || p.DV % 64 != 0) return hipErrorInvalidValue;
  switch (p.DK) {
    case 64: return launch_dk<64>(p, sig, stream);
    case 128: return launch_dk<128>(p, sig, stream);
    case 256: return launch_dk<256>(p, sig, stream);
    case 512: return launch_dk<512>(p, sig, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mlstm
