// Backward pass of the chunkwise mLSTM (gfx950): the gradients of <dH, H>
// with respect to Q, K, V, both gate pre-activations and the initial state.
//
// The pages print no backward pass.  What is computed is the derivative of
// the forward pass of "xLSTM: the NX-AI repository behind the extended LSTM
// architecture" (section "Exponential gating, matrix memory, and why the
// kernels decide everything"), organised chunk by chunk like the forward of
// "Tiled Flash Linear Attention: More Efficient Linear RNN and xLSTM
// Kernels" (abstract: chunkwise-parallel training).  The max-state m is a
// stabiliser and is held constant; with eps = 0 the output does not depend on
// it, so the gradient is exact.
//
// Per head, with s the query scale, b the in-chunk inclusive sum of
// log sigmoid(f), g its value at the chunk end, src = i (exp gate) or
// log sigmoid(i) (sig gate), M_c the stabiliser of the state entering chunk
// c, m_t and den_t the row max-state and stabilised normaliser of the
// forward pass, and z_t = max(|den_t|, e^{-m_t}) + eps:
//   dn_t    = dh_t / z_t                                  (sig: dh_t)
//   delta_t = -(dh_t . h_t) / z_t * sign(den_t) where |den_t| > e^{-m_t}, else 0
//   w_tj    = e^{b_t - b_j + src_j - m_t}   (j <= t in the same chunk; sig: no m_t)
//   dP_tj   = dn_t . v_j + delta_t
//   dq_t    = s sum_j w_tj dP_tj k_j + s e^{b_t + M_c - m_t} (C_c dn_t + delta_t n_c)
//   dk_j    = s sum_t w_tj dP_tj q_t + e^{g - b_j + src_j - M_{c+1}} (G_c v_j + N_c)
//   dv_j    = sum_t w_tj s (q_t . k_j) dn_t + e^{g - b_j + src_j - M_{c+1}} G_c^T k_j
// (C_c, n_c) is the forward state entering chunk c, and (G_c, N_c) the
// gradient that every later query sends into the state after chunk c, kept
// relative to that state's stabiliser:
//   G_{c-1} = e^{M_c + g_c - M_{c+1}} G_c + s sum_{t in c} e^{b_t + M_c - m_t} q_t dn_t^T
//   N_{c-1} = the same with delta_t in place of dn_t,   (G_{-1}, N_{-1}) = (dC0, dn0)
// (sig gate: no stabilisers, no N).  Every exponent above is <= 0.  The gate
// gradients follow from two identities of the exact gradient:
//   d i_j = k_j . dk_j                 (sig gate: times sigmoid(-i_j))
//   d f_t = sigmoid(-f_t) sum_{u >= t} (q_u . dq_u - k_u . dk_u)
// and dm0 = sum(dC0 * C0) + dn0 . n0.
//
// Kernels, 256 threads each; with float32 inputs on fp32 matrix cores
// (v_mfma_f32_16x16x4_f32: exact products of float32 operands), with bf16
// inputs on bf16 matrix cores with computed operands split (below):
//   bw_prep    per position: b, src, and 1/z, delta unless the recompute
//              formed them
//   bw_dstate  the reverse recurrence of (G, N): one workgroup per head and
//              64 x 64 tile of G, chunks in reverse order; G_c goes to HBM
//              (the row-tile variant writes it in the packed bf16 hi + lo
//              layout of the chunk states, which dk and dv then stage as is)
//   bw_tiles   dq per 64-query tile, dk and dv per 64-key tile: the inter-
//              chunk term first, then for each causal partner tile the
//              64 x 64 score tile (dP or the raw scores), weighted in
//              registers and fed straight back to the matrix cores as the
//              operand of the output product
//   bw_gates   the reverse scan of q.dq - k.dk over the sequence, d_i, dm0
// Matrix-core fragment of v_mfma_f32_16x16x4_f32: lane l supplies
// A[l % 16][l / 16] and B[l / 16][l % 16]; the 16 x 16 accumulator holds in
// lane l register r the element (4 (l / 16) + r, l % 16).  An accumulator
// tile is therefore a ready B operand of a product that contracts over its
// rows: in step r the lanes' slot l / 16 stands for row 4 (l / 16) + r.
#include "device_common.h"
#include "tile_order.h"
#include "kernels.h"

namespace mlstm {
namespace {

constexpr int kT = 64;    // rows of a tile
constexpr int kLdA = 68;  // LDS row stride (floats) of tiles read with the row on lane % 16
constexpr int kLdB = 80;  // LDS row stride of tiles read with the row on lane / 16

enum { kModeDQ = 0, kModeDK = 1, kModeDV = 2 };

__device__ __forceinline__ float4_t mma4(float a, float b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float sigmoid_neg(float x) { return 1.0f / (1.0f + expf(x)); }

// 16 consecutive values at element offset `off` of a bf16 or float32 array.
__device__ __forceinline__ void load16(const void* base, bool bf16, size_t off, float (&x)[16]) {
  if (bf16) {
    const uint4* q = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
    const uint4 a = q[0], b = q[1];
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    const float4* q = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 v = q[i];
      x[4 * i] = v.x;
      x[4 * i + 1] = v.y;
      x[4 * i + 2] = v.z;
      x[4 * i + 3] = v.w;
    }
  }
}

// LDS tile dst[r * ld + c] (r, c < 64) = rowscale[r] * src[(row0 + r) * D + col0 + c]
// for r < nrows, zero below.  256 threads: thread t fills row t / 4,
// columns 16 (t % 4) .. 16 (t % 4) + 15.
__device__ __forceinline__ void stage_tile(float* dst, int ld, const void* src, bool bf16, size_t row0, int D,
                                           int col0, int nrows, const float* rowscale) {
  const int r = threadIdx.x >> 2, c = (threadIdx.x & 3) * 16;
  float x[16];
  if (r < nrows) {
    load16(src, bf16, (row0 + r) * (size_t)D + col0 + c, x);
    if (rowscale) {
      const float sc = rowscale[r];
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] *= sc;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = 0.0f;
  }
  float4* d = reinterpret_cast<float4*>(dst + r * ld + c);
#pragma unroll
  for (int i = 0; i < 4; ++i) d[i] = make_float4(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
}

// ---------------------------------------------------------------------------
// Per-position terms: b (in-chunk inclusive sum of log sigmoid(f)), src, and
// for the exp gate 1/z and delta.  One workgroup per (head, chunk).
template <bool SIG>
__global__ __launch_bounds__(256) void bw_prep_kernel(const BwParams p) {
  __shared__ float s_tot[4];
  const int bh = blockIdx.x / p.Nc, c = blockIdx.x % p.Nc;
  const int t0 = c * p.L, Lc = min(p.L, p.S - t0);
  const size_t rb = (size_t)bh * p.S + t0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int pos = 4 * tid + e;
    v[e] = pos < Lc ? log_sigmoid(p.f_pre[rb + pos]) : 0.0f;
  }
  block_scan4<false, 4>(v, s_tot);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int pos = 4 * tid + e;
    if (pos < Lc) {
      p.gb[rb + pos] = v[e];
      const float ip = p.i_pre[rb + pos];
      p.gsrc[rb + pos] = SIG ? log_sigmoid(ip) : ip;
    }
  }
  // exp gate: 1/z and delta, unless the recompute formed them
  if (!SIG && !p.delta_ready) {
    // float32 dH on 16-byte boundaries: 16-byte loads, the row's pieces all
    // in flight at once
    const bool vec = !p.dh_bf16 && (p.DV & 255) == 0 && (reinterpret_cast<uintptr_t>(p.dH) & 15) == 0;
    for (int r = wave; r < Lc; r += 4) {
      const size_t row = rb + r;
      float d = 0.0f;
      if (vec) {
        const float4* a = reinterpret_cast<const float4*>(static_cast<const float*>(p.dH) + row * p.DV);
        const float4* b = reinterpret_cast<const float4*>(p.H + row * p.DV);
        for (int e = lane; e < p.DV / 4; e += 64) {
          const float4 x = a[e], y = b[e];
          d += x.x * y.x + x.y * y.y + x.z * y.z + x.w * y.w;
        }
      } else {
        for (int e = lane; e < p.DV; e += 64) {
          const size_t i = row * p.DV + e;
          const float dh = p.dh_bf16 ? bf16_to_f32(static_cast<const uint16_t*>(p.dH)[i])
                                     : static_cast<const float*>(p.dH)[i];
          d += dh * p.H[i];
        }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) d += __shfl_xor(d, o, 64);
      if (lane == 0) {
        const float den = p.den_rows[row], em = expf(-p.m_rows[row]);
        const float invz = 1.0f / (fmaxf(fabsf(den), em) + p.eps);
        p.ginvz[row] = invz;
        p.gdelta[row] = fabsf(den) > em ? (den > 0.0f ? -d * invz : d * invz) : 0.0f;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Reverse recurrence of the state gradient (G, N).  Grid (BH, DK/64, DV/64);
// wave w holds rows 16w .. 16w+15 of the 64 x 64 tile of G.  Entry c of
// dC_states is G_c (the gradient into the state after chunk c), entry Nc-1 is
// zero; the value left after chunk 0 is dC0.
template <bool SIG>
__global__ __launch_bounds__(256) void bw_dstate_kernel(const BwParams p) {
  __shared__ __align__(16) float s_q[kT * kLdB];  // [t][k]
  __shared__ __align__(16) float s_b[kT * kLdB];  // [t][v]: weighted dn
  __shared__ float s_w[kT], s_wd[kT];
  const int bh = blockIdx.x, kt = blockIdx.y, vt = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g4 = lane >> 4, l16 = lane & 15;
  const int DK = p.DK, DV = p.DV, Nc = p.Nc;
  const bool own_n = !SIG && vt == 0;
  float4_t acc[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) acc[nb] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float dn = 0.0f;
  for (int c = Nc - 1; c >= 0; --c) {
    float* G = p.dC_states + ((size_t)bh * Nc + c) * DK * DV;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        G[(size_t)(kt * kT + 16 * wave + 4 * g4 + r) * DV + vt * kT + 16 * nb + l16] = acc[nb][r];
    if (own_n && tid < kT) p.dn_states[((size_t)bh * Nc + c) * DK + kt * kT + tid] = dn;

    const int t0 = c * p.L, Lc = min(p.L, p.S - t0);
    const size_t rb = (size_t)bh * p.S + t0;
    const float g = p.gb[rb + Lc - 1];
    float Min = 0.0f, decay;
    if constexpr (SIG) {
      decay = expf(g);
    } else {
      Min = p.m_states[(size_t)bh * (Nc + 1) + c];
      decay = expf(Min + g - p.m_states[(size_t)bh * (Nc + 1) + c + 1]);
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[nb] *= decay;
    dn *= decay;

    for (int ts = 0; ts < Lc; ts += kT) {
      const int nr = min(kT, Lc - ts);
      if (tid < kT) {
        float w = 0.0f, wd = 0.0f;
        if (tid < nr) {
          const size_t r = rb + ts + tid;
          if constexpr (SIG) {
            w = p.scale * expf(p.gb[r]);
          } else {
            const float e = p.scale * expf(p.gb[r] + Min - p.m_rows[r]);
            w = e * p.ginvz[r];
            wd = e * p.gdelta[r];
          }
        }
        s_w[tid] = w;
        s_wd[tid] = wd;
      }
      __syncthreads();
      stage_tile(s_q, kLdB, p.Q, p.qkv_bf16, rb + ts, DK, kt * kT, nr, nullptr);
      stage_tile(s_b, kLdB, p.dH, p.dh_bf16, rb + ts, DV, vt * kT, nr, s_w);
      __syncthreads();
#pragma unroll 4
      for (int j = 0; j < 16; ++j) {
        const int t = 4 * j + g4;
        const float a = s_q[t * kLdB + 16 * wave + l16];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[nb] = mma4(a, s_b[t * kLdB + 16 * nb + l16], acc[nb]);
      }
      if (own_n && tid < kT)
        for (int t = 0; t < nr; ++t) dn += s_wd[t] * s_q[t * kLdB + tid];
      __syncthreads();
    }
  }
  if (p.dC0) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        p.dC0[(size_t)bh * DK * DV + (size_t)(kt * kT + 16 * wave + 4 * g4 + r) * DV + vt * kT + 16 * nb + l16] =
            acc[nb][r];
  }
  if (own_n && p.dn0 && tid < kT) p.dn0[(size_t)bh * DK + kt * kT + tid] = dn;
}

// ---------------------------------------------------------------------------
// Gate terms of 64 rows of a chunk (zero past the chunk end).
struct RowGates {
  float b[kT], src[kT], m[kT], invz[kT], delta[kT];
};

template <bool SIG>
__device__ __forceinline__ void load_rows(RowGates& g, const BwParams& p, size_t rb, int r0, int Lc) {
  const int t = threadIdx.x;
  if (t < kT) {
    const bool ok = r0 + t < Lc;
    const size_t r = rb + r0 + t;
    g.b[t] = ok ? p.gb[r] : 0.0f;
    g.src[t] = ok ? p.gsrc[r] : 0.0f;
    if constexpr (!SIG) {
      g.m[t] = ok ? p.m_rows[r] : 0.0f;
      g.invz[t] = ok ? p.ginvz[r] : 0.0f;
      g.delta[t] = ok ? p.gdelta[r] : 0.0f;
    }
  }
}

// dq (MODE kModeDQ, own rows = 64 queries), dk (kModeDK) or dv (kModeDV,
// own rows = 64 keys) for one 64-row tile of one chunk and W = 16 NY output
// columns.  Wave w owns rows 16w .. 16w+15 of the tile: they are the columns
// of its accumulators, which hold the transposed output (out^T[y][own]).
template <int MODE, bool SIG, int NY>
__global__ __launch_bounds__(256) void bw_tiles_kernel(const BwParams p) {
  constexpr int W = 16 * NY;
  __shared__ __align__(16) float s_x[kT * kLdA];  // partner tile, contraction chunk  [o][x]
  __shared__ __align__(16) float s_w[kT * kLdA];  // own tile, contraction chunk     [w][x]
  __shared__ __align__(16) float s_y[kT * kLdB];  // output-side operand chunk
  __shared__ RowGates g_own, g_oth;

  const int nT = p.L / kT;
  const TileIdx ti = xcd_tile();
  const int ot = ti.x % nT;
  const int rest = ti.x / nT;
  const int c = rest % p.Nc, bh = rest / p.Nc;
  const int t0 = c * p.L, Lc = min(p.L, p.S - t0);
  const int own0 = ot * kT;
  if (own0 >= Lc) return;
  const int nown = min(kT, Lc - own0);
  const size_t rb = (size_t)bh * p.S + t0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g4 = lane >> 4, l16 = lane & 15;
  const int DK = p.DK, DV = p.DV, Nc = p.Nc;
  const int DO = MODE == kModeDV ? DV : DK;  // output width
  const int y0 = ti.y * W;
  const bool qb = p.qkv_bf16, hb = p.dh_bf16;

  load_rows<SIG>(g_own, p, rb, own0, Lc);
  __syncthreads();
  const int w = 16 * wave + l16;  // own row of this lane's accumulator columns
  const bool own_ok = w < nown;
  const float ob = g_own.b[w], osrc = g_own.src[w];
  const float om = SIG ? 0.0f : g_own.m[w];
  const float odelta = SIG ? 0.0f : g_own.delta[w];
  const float gc = p.gb[rb + Lc - 1];

  float4_t acc[NY];
#pragma unroll
  for (int i = 0; i < NY; ++i) acc[i] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // ---- inter-chunk term
  if constexpr (MODE == kModeDQ) {
    // (C_c dn)^T: contraction over v; then times e^{b + M_c - m}, plus delta n_c
    if (c > 0 || p.C0 || p.n0) {
      const float* Cst = p.C_states + ((size_t)bh * (Nc + 1) + c) * DK * DV;
      for (int e0 = 0; e0 < DV; e0 += kT) {
        __syncthreads();
        stage_tile(s_w, kLdA, p.dH, hb, rb + own0, DV, e0, nown, SIG ? nullptr : g_own.invz);
        for (int yc = 0; yc < W / kT; ++yc) {
          __syncthreads();
          stage_tile(s_x, kLdA, Cst, false, y0 + yc * kT, DV, e0, kT, nullptr);  // [d][e]
          __syncthreads();
#pragma unroll 4
          for (int j = 0; j < 16; ++j) {
            const float b = s_w[w * kLdA + 4 * j + g4];
#pragma unroll
            for (int yb = 0; yb < 4; ++yb)
              acc[4 * yc + yb] = mma4(s_x[(16 * yb + l16) * kLdA + 4 * j + g4], b, acc[4 * yc + yb]);
          }
        }
      }
      float wq;
      if constexpr (SIG) wq = own_ok ? expf(ob) : 0.0f;
      else wq = own_ok ? expf(ob + p.m_states[(size_t)bh * (Nc + 1) + c] - om) : 0.0f;
      const float* nst = SIG ? nullptr : p.n_states + ((size_t)bh * (Nc + 1) + c) * DK;
#pragma unroll
      for (int yb = 0; yb < NY; ++yb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float x = acc[yb][r] * wq;
          if constexpr (!SIG) x += odelta * wq * nst[y0 + 16 * yb + 4 * g4 + r];
          acc[yb][r] = x;
        }
    }
  } else {
    if (c < Nc - 1) {
      // dk: (G v + N)^T, contraction over v;  dv: (G^T k)^T, contraction over k
      const float* G = p.dC_states + ((size_t)bh * Nc + c) * DK * DV;
      const int XD = MODE == kModeDK ? DV : DK;
      for (int x0 = 0; x0 < XD; x0 += kT) {
        __syncthreads();
        if constexpr (MODE == kModeDK) stage_tile(s_w, kLdA, p.V, qb, rb + own0, DV, x0, nown, nullptr);
        else stage_tile(s_w, kLdA, p.K, qb, rb + own0, DK, x0, nown, nullptr);
        for (int yc = 0; yc < W / kT; ++yc) {
          __syncthreads();
          if constexpr (MODE == kModeDK) stage_tile(s_y, kLdA, G, false, y0 + yc * kT, DV, x0, kT, nullptr);  // [d][v]
          else stage_tile(s_y, kLdB, G, false, x0, DV, y0 + yc * kT, kT, nullptr);  // [k][e]
          __syncthreads();
#pragma unroll 4
          for (int j = 0; j < 16; ++j) {
            const float b = s_w[w * kLdA + 4 * j + g4];
#pragma unroll
            for (int yb = 0; yb < 4; ++yb) {
              const float a = MODE == kModeDK ? s_y[(16 * yb + l16) * kLdA + 4 * j + g4]
                                              : s_y[(4 * j + g4) * kLdB + 16 * yb + l16];
              acc[4 * yc + yb] = mma4(a, b, acc[4 * yc + yb]);
            }
          }
        }
      }
      float wk;
      const float Mo = SIG ? 0.0f : p.m_states[(size_t)bh * (Nc + 1) + c + 1];
      wk = own_ok ? expf(gc - ob + osrc - Mo) : 0.0f;
      if constexpr (MODE == kModeDK) {
        const float* Nst = SIG ? nullptr : p.dn_states + ((size_t)bh * Nc + c) * DK;
        const float f = wk / p.scale;
#pragma unroll
        for (int yb = 0; yb < NY; ++yb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float x = acc[yb][r];
            if constexpr (!SIG) x += Nst[y0 + 16 * yb + 4 * g4 + r];
            acc[yb][r] = x * f;
          }
      } else {
#pragma unroll
        for (int yb = 0; yb < NY; ++yb) acc[yb] *= wk;
      }
    }
  }

  // ---- intra-chunk term: every causal partner tile
  const int lo = MODE == kModeDQ ? 0 : ot;
  const int hi = MODE == kModeDQ ? ot : (Lc - 1) / kT;
  for (int xt = lo; xt <= hi; ++xt) {
    const int x0 = xt * kT, nx = min(kT, Lc - x0);
    __syncthreads();
    load_rows<SIG>(g_oth, p, rb, x0, Lc);
    float4_t sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    const int XD = MODE == kModeDV ? DK : DV;
    for (int c0 = 0; c0 < XD; c0 += kT) {
      __syncthreads();
      if constexpr (MODE == kModeDQ) {
        stage_tile(s_x, kLdA, p.V, qb, rb + x0, DV, c0, nx, nullptr);
        stage_tile(s_w, kLdA, p.dH, hb, rb + own0, DV, c0, nown, SIG ? nullptr : g_own.invz);
      } else if constexpr (MODE == kModeDK) {
        stage_tile(s_x, kLdA, p.dH, hb, rb + x0, DV, c0, nx, SIG ? nullptr : g_oth.invz);
        stage_tile(s_w, kLdA, p.V, qb, rb + own0, DV, c0, nown, nullptr);
      } else {
        stage_tile(s_x, kLdA, p.Q, qb, rb + x0, DK, c0, nx, nullptr);
        stage_tile(s_w, kLdA, p.K, qb, rb + own0, DK, c0, nown, nullptr);
      }
      __syncthreads();
#pragma unroll 4
      for (int j = 0; j < 16; ++j) {
        const float b = s_w[w * kLdA + 4 * j + g4];
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[i] = mma4(s_x[(16 * i + l16) * kLdA + 4 * j + g4], b, sc[i]);
      }
    }
    // weights: sc[i][r] is the partner row o = 16 i + 4 g4 + r against own row w
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int o = 16 * i + 4 * g4 + r;
        float x = 0.0f;
        if constexpr (MODE == kModeDQ) {
          // o = key, w = query
          if (own_ok && o < nx && x0 + o <= own0 + w) {
            const float ex = ob - g_oth.b[o] + g_oth.src[o] - om;
            x = expf(ex) * (sc[i][r] + odelta);
          }
        } else {
          // o = query, w = key
          if (own_ok && o < nx && own0 + w <= x0 + o) {
            const float ex = g_oth.b[o] - ob + osrc - (SIG ? 0.0f : g_oth.m[o]);
            if constexpr (MODE == kModeDK) x = expf(ex) * (sc[i][r] + (SIG ? 0.0f : g_oth.delta[o]));
            else x = expf(ex) * p.scale * sc[i][r];
          }
        }
        sc[i][r] = x;
      }
    // output product: out^T[y][w] += sum_o Y[o][y] sc[o][w]
    for (int yc = 0; yc < W / kT; ++yc) {
      __syncthreads();
      if constexpr (MODE == kModeDQ) stage_tile(s_y, kLdA, p.K, qb, rb + x0, DK, y0 + yc * kT, nx, nullptr);
      else if constexpr (MODE == kModeDK) stage_tile(s_y, kLdA, p.Q, qb, rb + x0, DK, y0 + yc * kT, nx, nullptr);
      else stage_tile(s_y, kLdA, p.dH, hb, rb + x0, DV, y0 + yc * kT, nx, SIG ? nullptr : g_oth.invz);
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int o = 16 * i + 4 * g4 + r;
#pragma unroll
          for (int yb = 0; yb < 4; ++yb)
            acc[4 * yc + yb] = mma4(s_y[o * kLdA + 16 * yb + l16], sc[i][r], acc[4 * yc + yb]);
        }
    }
  }

  // ---- epilogue: scale, store, and q.dq / k.dk for the gate gradients
  const float fin = MODE == kModeDV ? 1.0f : p.scale;
  float* out = MODE == kModeDQ ? p.dQ : MODE == kModeDK ? p.dK : p.dV;
  float dot = 0.0f;
  if (own_ok) {
    const size_t orow = rb + own0 + w;
#pragma unroll
    for (int yb = 0; yb < NY; ++yb) {
      const int y = y0 + 16 * yb + 4 * g4;
      const float4 o4 = make_float4(acc[yb][0] * fin, acc[yb][1] * fin, acc[yb][2] * fin, acc[yb][3] * fin);
      *reinterpret_cast<float4*>(out + orow * DO + y) = o4;
      if constexpr (MODE != kModeDV) {
        const void* src = MODE == kModeDQ ? p.Q : p.K;
        float x[4];
        if (qb) {
          const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(src) + orow * DK + y);
          x[0] = __uint_as_float(u.x << 16);
          x[1] = __uint_as_float(u.x & 0xffff0000u);
          x[2] = __uint_as_float(u.y << 16);
          x[3] = __uint_as_float(u.y & 0xffff0000u);
        } else {
          const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(src) + orow * DK + y);
          x[0] = v.x;
          x[1] = v.y;
          x[2] = v.z;
          x[3] = v.w;
        }
        dot += x[0] * o4.x + x[1] * o4.y + x[2] * o4.z + x[3] * o4.w;
      }
    }
  }
  if constexpr (MODE != kModeDV) {
    dot += __shfl_xor(dot, 16, 64);
    dot += __shfl_xor(dot, 32, 64);
    if (g4 == 0 && own_ok) (MODE == kModeDQ ? p.qdq : p.kdk)[rb + own0 + w] = dot;
  }
}

// ---------------------------------------------------------------------------
// The same three modes for bf16 inputs on bf16 matrix cores
// (v_mfma_f32_16x16x32_bf16: lane l supplies A[l % 16][8 (l / 16) + e] and
// B[8 (l / 16) + e][l % 16], e = 0..7).  Q, K and V enter unchanged; every
// operand computed in float32 (dH / z, the states, the weighted score tiles)
// is carried as a bf16 hi + lo pair, so a product with one computed side
// takes two passes and one with two computed sides three (hi.hi + hi.lo +
// lo.hi).  LDS tiles hold bf16 bits, row stride kLd16.  The output product
// reads its A operand from a row-major tile [partner row][y] with transposing
// reads (frag16_tr); its B operand
// is the pair of score accumulators (partner blocks 2p, 2p+1) split to bf16:
// slot e stands for partner row 32 p + 16 (e / 4) + 4 (l / 16) + e % 4.
constexpr int kLd16 = 72;

// The transpose: dst[c * kLd16 + r] for source row r, column c.
__device__ __forceinline__ void stage_cols16(uint16_t* hi, uint16_t* lo, const void* src, bool bf16, size_t row0,
                                             int D, int col0, int nrows, const float* rowscale) {
  const int r = threadIdx.x >> 2, c = (threadIdx.x & 3) * 16;
  float x[16];
  if (r < nrows) {
    load16(src, bf16, (row0 + r) * (size_t)D + col0 + c, x);
    const float sc = rowscale ? rowscale[r] : 1.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] *= sc;
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = 0.0f;
  }
#pragma unroll
  for (int i = 0; i < 16; i += 2) {
    uint32_t hw, lw;
    split_bf16x2(x[i], x[i + 1], hw, lw);
    hi[(c + i) * kLd16 + r] = (uint16_t)(hw & 0xffff);
    hi[(c + i + 1) * kLd16 + r] = (uint16_t)(hw >> 16);
    if (lo) {
      lo[(c + i) * kLd16 + r] = (uint16_t)(lw & 0xffff);
      lo[(c + i + 1) * kLd16 + r] = (uint16_t)(lw >> 16);
    }
  }
}

__device__ __forceinline__ bf16x8_t frag16(const uint16_t* t, int row, int k0) {
  return as_bf16x8(*reinterpret_cast<const uint4*>(t + row * kLd16 + k0));
}

// A fragment (lane l supplies row l % 16 of A, slots e = 0..7) read from a
// row-major LDS tile X whose rows run along A's contraction axis: slots 0..3
// from rows r0 .. r0+3 and slots 4..7 from rows r0+dr .. r0+dr+3, all at
// column c0 + l % 16 (r0 carries the lane group's offset).  Two transposing
// reads, ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives
// element e from address a_{i/4 + 4e} + i % 4, a_j the address lane j gives;
// lane j gives row r0 + j / 4, columns c0 + 4 (j % 4) .. + 3.  So the tile
// is written with row stores (16 bytes) rather than transposing ones.
__device__ __forceinline__ bf16x8_t frag16_tr(const uint16_t* X, int r0, int dr, int c0) {
  const int j = threadIdx.x & 15;
  const uint16_t* base = X + (r0 + (j >> 2)) * kLd16 + c0 + 4 * (j & 3);
  typedef short s4_t __attribute__((ext_vector_type(4)));
  const s4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4_t*)(base));
  const s4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4_t*)(base + dr * kLd16));
  const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
  return as_bf16x8(make_uint4(a.x, a.y, b.x, b.y));
}

// The state-gradient recurrence on bf16 matrix cores (bf16 inputs): per
// 64-position stage, G[k][v] += sum_t Q[t][k] W[t][v] with W = s e^{b + M - m}
// dn the computed operand; both sides are staged transposed ([k][t] and
// [v][t], W as hi + lo), so the contraction over t runs along LDS rows.
template <bool SIG>
__global__ __launch_bounds__(256) void bw_dstate16_kernel(const BwParams p) {
  __shared__ __align__(16) uint16_t s_qt[kT * kLd16];     // Q^T [k][t]
  __shared__ __align__(16) uint16_t s_wt[2][kT * kLd16];  // W^T [v][t] (hi, lo)
  __shared__ float s_w[kT], s_wd[kT];
  const int bh = blockIdx.x, kt = blockIdx.y, vt = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g4 = lane >> 4, l16 = lane & 15;
  const int DK = p.DK, DV = p.DV, Nc = p.Nc;
  const bool own_n = !SIG && vt == 0;
  float4_t acc[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) acc[nb] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float dn = 0.0f;
  for (int c = Nc - 1; c >= 0; --c) {
    float* G = p.dC_states + ((size_t)bh * Nc + c) * DK * DV;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        G[(size_t)(kt * kT + 16 * wave + 4 * g4 + r) * DV + vt * kT + 16 * nb + l16] = acc[nb][r];
    if (own_n && tid < kT) p.dn_states[((size_t)bh * Nc + c) * DK + kt * kT + tid] = dn;

    const int t0 = c * p.L, Lc = min(p.L, p.S - t0);
    const size_t rb = (size_t)bh * p.S + t0;
    const float g = p.gb[rb + Lc - 1];
    float Min = 0.0f, decay;
    if constexpr (SIG) {
      decay = expf(g);
    } else {
      Min = p.m_states[(size_t)bh * (Nc + 1) + c];
      decay = expf(Min + g - p.m_states[(size_t)bh * (Nc + 1) + c + 1]);
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[nb] *= decay;
    dn *= decay;

    for (int ts = 0; ts < Lc; ts += kT) {
      const int nr = min(kT, Lc - ts);
      if (tid < kT) {
        float w = 0.0f, wd = 0.0f;
        if (tid < nr) {
          const size_t r = rb + ts + tid;
          if constexpr (SIG) {
            w = p.scale * expf(p.gb[r]);
          } else {
            const float e = p.scale * expf(p.gb[r] + Min - p.m_rows[r]);
            w = e * p.ginvz[r];
            wd = e * p.gdelta[r];
          }
        }
        s_w[tid] = w;
        s_wd[tid] = wd;
      }
      __syncthreads();
      stage_cols16(s_qt, nullptr, p.Q, true, rb + ts, DK, kt * kT, nr, nullptr);
      stage_cols16(s_wt[0], s_wt[1], p.dH, p.dh_bf16, rb + ts, DV, vt * kT, nr, s_w);
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int k0 = 32 * j + 8 * g4;
        const bf16x8_t a = frag16(s_qt, 16 * wave + l16, k0);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          acc[nb] = mma16b(a, frag16(s_wt[0], 16 * nb + l16, k0), acc[nb]);
          acc[nb] = mma16b(a, frag16(s_wt[1], 16 * nb + l16, k0), acc[nb]);
        }
      }
      if (own_n && tid < kT)
        for (int t = 0; t < nr; ++t) dn += s_wd[t] * __uint_as_float((uint32_t)s_qt[tid * kLd16 + t] << 16);
      __syncthreads();
    }
  }
  if (p.dC0) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        p.dC0[(size_t)bh * DK * DV + (size_t)(kt * kT + 16 * wave + 4 * g4 + r) * DV + vt * kT + 16 * nb + l16] =
            acc[nb][r];
  }
  if (own_n && p.dn0 && tid < kT) p.dn0[(size_t)bh * DK + kt * kT + tid] = dn;
}

// Row-tile form of the (G, N) recurrence for bf16 Q: a workgroup of eight
// waves keeps a TK x TV tile of G (each wave a 64 x 64 block on the 32x32x16
// matrix cores) while it walks the chunks from last to first.  Each block of
// weighted dH rows is then staged once for all TK key rows, and each Q block
// once for all TV value columns.  With TV < DHV (256 x 128 tiles for float32
// dH) every workgroup reads only its own columns of dH, the largest input,
// and the workgroups of a head share the Q rows instead.  Per chunk c: G (packed hi + lo) and N
// leave for slot c, are decayed by the chunk's gate and gain the chunk's sums
//   G += Q^T (w . dH),  N += Q^T wd,
// w_t = s e^{b_t + M_c - m_t} / z_t and wd_t the same with delta_t (sig gate:
// w_t = s e^{b_t}, no N).  Q enters the matrix cores as raw bf16 (exact);
// w . dH is split into bf16 hi + lo.  Software pipeline over TB-row blocks
// of the flattened (chunk, block) sequence, as in the forward state kernel:
// two LDS stages and one barrier per block, global loads two blocks ahead.
// A block of float32 dH is 16 rows on the 512-column tiles, so that both
// register sets of its loads fit beside the accumulators (a spilled
// register would be reloaded through the same in-order counter as the loads
// in flight, and wait for them); on the 128-column tiles 32 rows fit.
// Staging: the lanes of wave x are split evenly over its time rows
// (TB / 8 rows each; a row's owner lanes hold its Q pieces and gate terms),
// and the same wave stages those rows of dH, taking each row's weight from
// the row's first owner lane.
template <int TK, int TV, int TB, bool SIG, bool DHB>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void bw_dstate_rows_kernel(
    const BwParams p) {
  constexpr int NT = 512, NW = 8;
  constexpr int NWC = TV / 64;
  static_assert((TK / 64) * NWC == NW, "eight 64x64 wave tiles");
  constexpr int LDK = TK + 32, LDV = TV + 32;  // transposing reads: 16 banks mod 64
  constexpr int RW = TB / NW;                  // time rows per wave
  constexpr int EPT = TB * TK / NT;            // Q elements per thread and block
  constexpr int TPR = TK / EPT;                // staging lanes per time row
  static_assert((TB == 16 || TB == 32) && RW * TPR == 64, "staging split");
  static_assert(EPT == 2 || EPT == 4 || EPT == 8 || EPT == 16, "Q pieces of 4, 8, 16 or 32 bytes");
  constexpr int VE = DHB ? 8 : 4;       // dH elements per 16-byte load
  constexpr int VSEG = TV / VE;         // 16-byte pieces per dH row
  constexpr int VPT = RW * VSEG / 64;   // pieces per lane and block
  static_assert(VPT * 64 == RW * VSEG && VPT >= 1, "dH staging split");
  constexpr int QBUF = TB * LDK, WBUF = TB * LDV;
  struct alignas(16) Uint4x2 {
    uint4 a, b;
  };
  typedef typename std::conditional<
      EPT == 2, uint32_t,
      typename std::conditional<EPT == 4, uint2, typename std::conditional<EPT == 8, uint4, Uint4x2>::type>::type>::type
      QVec;

  __shared__ float s_np[NW][TK];
  __shared__ __align__(16) uint16_t s_q[2 * QBUF];
  __shared__ __align__(16) uint16_t s_wh[2 * WBUF];
  __shared__ __align__(16) uint16_t s_wl[2 * WBUF];

  const int NTK = p.DK / TK, NTV = p.DV / TV;
  const int nblk = gridDim.x;
  int bid = blockIdx.x;
  // the tiles of one head (and segment) on one XCD: they read the same Q or
  // dH rows
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int vt = bid % NTV;
  const int kt = (bid / NTV) % NTK;
  const int seg = (bid / (NTV * NTK)) % p.nseg;
  const int bh = bid / (NTV * NTK * p.nseg);
  const bool n_out = vt == 0;  // N is the same for every column slice
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h2 = lane >> 5, l32 = lane & 31;
  const int S = p.S, DK = p.DK, L = p.L, Nc = p.Nc;
  // chunks [c_beg, c_end) of this segment, walked from the last; a segment
  // other than the last starts from a zero state gradient and the join
  // kernels add what enters it from the later segments
  const int c_beg = p.nseg > 1 ? seg * p.cps : 0;
  const int c_end = p.nseg > 1 ? min(Nc, c_beg + p.cps) : Nc;
  const int DV = p.DV;
  const int wr0 = (wave / NWC) * 64, wc0 = (wave % NWC) * 64;
  const int vc0 = vt * TV;  // first value column of the slice
  const size_t gbase = (size_t)bh * S;
  const int krs = tid / TPR, kcs = (tid % TPR) * EPT;  // own time row (RW wave + lane / TPR) and columns

  float16_t acc[2][2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rb][cb][r] = 0.0f;
  float nreg = 0.0f;  // N for key row kt * TK + tid (tid < TK)

  // Q and dH of this head through buffer resources; a block's first row is
  // added to the lane offset, so rows past the sequence fall outside the
  // range check and read as zero.
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(static_cast<const uint16_t*>(p.Q) + gbase * DK + kt * TK,
                                              (uint32_t)(((size_t)S * DK - kt * TK) * 2));
  const __amdgpu_buffer_rsrc_t rd =
      make_rsrc(static_cast<const char*>(p.dH) + gbase * DV * (DHB ? 2 : 4), (uint32_t)((size_t)S * DV * (DHB ? 2 : 4)));
  const int qvoff = (krs * DK + kcs) * 2;

  // block gi: chunk c_end - 1 - gi / BPC, rows [tb, tb + TB) of it; blocks
  // past the end of a short last chunk read zeros and carry weight zero
  const int BPC = L / TB;
  const int NBLK = (c_end - c_beg) * BPC;

  QVec qr[2];
  uint4 dr[2][VPT];
  float gbr[2], mr[2], izr[2], dlr[2];  // own row's gate terms
  float glr[2], Mcr[2], Mnr[2];         // chunk scalars (first block of a chunk)
  auto load_blk = [&](auto set, int gi) {
    constexpr int s = decltype(set)::value;
    const int c = c_end - 1 - gi / BPC, tb = (gi % BPC) * TB;
    const int t0 = c * L, Lc = min(L, S - t0);
    const int trow = t0 + tb;
    const int qo = qvoff + trow * DK * 2;
    if constexpr (EPT == 2) {
      qr[s] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rq, qo, 0, 0);
    } else if constexpr (EPT == 4) {
      const v2i32_t q2 = __builtin_amdgcn_raw_buffer_load_b64(rq, qo, 0, 0);
      qr[s] = make_uint2((uint32_t)q2.x, (uint32_t)q2.y);
    } else if constexpr (EPT == 8) {
      qr[s] = buf_load16(rq, qo);
    } else {
      qr[s].a = buf_load16(rq, qo);
      qr[s].b = buf_load16(rq, qo + 16);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int f = i * 64 + lane, row = RW * wave + f / VSEG, seg = f % VSEG;
      dr[s][i] = buf_load16_nt(rd, ((trow + row) * DV + vc0 + seg * VE) * (DHB ? 2 : 4));
    }
    const int t = trow + krs;
    const bool ok = t < S;
    gbr[s] = ok ? p.gb[gbase + t] : 0.0f;
    if constexpr (!SIG) {
      mr[s] = ok ? p.m_rows[gbase + t] : 0.0f;
      izr[s] = ok ? p.ginvz[gbase + t] : 0.0f;
      dlr[s] = ok ? p.gdelta[gbase + t] : 0.0f;
    }
    if (tb == 0) {
      glr[s] = p.gb[gbase + t0 + Lc - 1];
      if constexpr (!SIG) {
        Mcr[s] = p.m_states[(size_t)bh * (Nc + 1) + c];
        Mnr[s] = p.m_states[(size_t)bh * (Nc + 1) + c + 1];
      }
    }
  };

  // N: partial sums of the staging lanes, reduced over the lanes that share
  // key columns, then (after a barrier) over the waves
  float np[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) np[e] = 0.0f;
  bool n_pend = false;
  float n_dec = 1.0f;
  float Mc_s = 0.0f, dec_s = 1.0f;  // scalars of the chunk being staged
  float dec_pend = 1.0f;            // handed to the matrix-core side
  auto flush_n = [&]() {
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
#pragma unroll
      for (int o = TPR; o < 64; o <<= 1) np[e] += __shfl_xor(np[e], o, 64);
    }
    if (lane < TPR) {
#pragma unroll
      for (int e = 0; e < EPT; ++e) s_np[wave][kcs + e] = np[e];
    }
#pragma unroll
    for (int e = 0; e < EPT; ++e) np[e] = 0.0f;
    n_pend = true;
    n_dec = dec_s;
  };
  auto finish_n = [&](float* dst) {
    if (tid < TK) {
      float sacc = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) sacc += s_np[w][tid];
      nreg = nreg * n_dec + sacc;
      if (dst && n_out) dst[kt * TK + tid] = nreg;
    }
    n_pend = false;
  };

  auto stage_blk = [&](auto set, int gi) {
    constexpr int s = decltype(set)::value;
    const int c = c_end - 1 - gi / BPC, tb = (gi % BPC) * TB;
    if (tb == 0) {
      if (!SIG && gi > 0) flush_n();
      if constexpr (SIG) {
        dec_s = expf(glr[s]);
      } else {
        Mc_s = Mcr[s];
        dec_s = expf(Mc_s + glr[s] - Mnr[s]);
      }
      dec_pend = dec_s;
    }
    const bool ok = c * L + tb + krs < S;
    float w = 0.0f, wd = 0.0f;
    if (ok) {
      if constexpr (SIG) {
        w = p.scale * expf(gbr[s]);
      } else {
        const float e = p.scale * expf(gbr[s] + Mc_s - mr[s]);
        w = e * izr[s];
        wd = e * dlr[s];
      }
    }
    // Q as raw bf16; N partial sums
    if constexpr (EPT == 16) {
      *reinterpret_cast<uint4*>(s_q + s * QBUF + krs * LDK + kcs) = qr[s].a;
      *reinterpret_cast<uint4*>(s_q + s * QBUF + krs * LDK + kcs + 8) = qr[s].b;
    } else {
      *reinterpret_cast<QVec*>(s_q + s * QBUF + krs * LDK + kcs) = qr[s];
    }
    if constexpr (!SIG) {
      uint32_t qw[EPT / 2];
      __builtin_memcpy(qw, &qr[s], sizeof(qw));
#pragma unroll
      for (int e = 0; e < EPT / 2; ++e) {
        np[2 * e] += wd * __uint_as_float(qw[e] << 16);
        np[2 * e + 1] += wd * __uint_as_float(qw[e] & 0xffff0000u);
      }
    }
    // w . dH as bf16 hi + lo; the row's weight from its owner lanes
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int f = i * 64 + lane, rw = f / VSEG, seg = f % VSEG;
      float wi;
      if constexpr (VSEG % 64 == 0) {
        wi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), TPR * ((i * 64) / VSEG)));
      } else {
        wi = __shfl(w, TPR * rw, 64);
      }
      float x[VE];
      const uint32_t u[4] = {dr[s][i].x, dr[s][i].y, dr[s][i].z, dr[s][i].w};
      if constexpr (DHB) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[2 * e] = __uint_as_float(u[e] << 16) * wi;
          x[2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u) * wi;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = __uint_as_float(u[e]) * wi;
      }
      uint32_t hw[VE / 2], lw[VE / 2];
#pragma unroll
      for (int e = 0; e < VE / 2; ++e) split_bf16x2(x[2 * e], x[2 * e + 1], hw[e], lw[e]);
      const int o = s * WBUF + (RW * wave + rw) * LDV + seg * VE;
      if constexpr (DHB) {
        *reinterpret_cast<uint4*>(s_wh + o) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        *reinterpret_cast<uint4*>(s_wl + o) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
      } else {
        *reinterpret_cast<uint2*>(s_wh + o) = make_uint2(hw[0], hw[1]);
        *reinterpret_cast<uint2*>(s_wl + o) = make_uint2(lw[0], lw[1]);
      }
    }
  };

  // matrix-core side
  // G_c in the packed hi + lo layout of the chunk states: each half of a
  // 32 x 32 accumulator is one fragment (16-row k step, 32-column block)
  auto write_g = [&](int c) {
    uint16_t* P = p.G_packed + ((size_t)bh * Nc + c) * DK * DV * 2;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          uint32_t hw[4], lw[4];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            split_bf16x2(acc[rb][cb][8 * half + 2 * q], acc[rb][cb][8 * half + 2 * q + 1], hw[q], lw[q]);
          const int kk = (kt * TK + wr0 + 32 * rb) / 16 + half, nb = (vc0 + wc0 + 32 * cb) / 32;
          typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
          __builtin_nontemporal_store(u32x4_t{hw[0], hw[1], hw[2], hw[3]},
                                      reinterpret_cast<u32x4_t*>(P + pack_frag_offset(kk, nb, 0, DV) + lane * 8));
          __builtin_nontemporal_store(u32x4_t{lw[0], lw[1], lw[2], lw[3]},
                                      reinterpret_cast<u32x4_t*>(P + pack_frag_offset(kk, nb, 1, DV) + lane * 8));
        }
  };
  auto mma_blk = [&](auto set, int gi) {
    constexpr int s = decltype(set)::value;
    const int c = c_end - 1 - gi / BPC, tb = (gi % BPC) * TB;
    if (tb == 0) {
      write_g(c);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) acc[rb][cb] *= dec_pend;
    }
    const int Lc = min(L, S - c * L);
#pragma unroll
    for (int ks = 0; ks < TB / 16; ++ks) {
      if (tb + 16 * ks >= Lc) break;  // uniform: padding only
      bf16x8_t a[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) a[rb] = as_bf16x8(frag_tr_u(s_q + s * QBUF, LDK, 16 * ks, wr0 + 32 * rb, lane));
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const bf16x8_t bh_ = as_bf16x8(frag_tr_u(s_wh + s * WBUF, LDV, 16 * ks, wc0 + 32 * cb, lane));
        const bf16x8_t bl_ = as_bf16x8(frag_tr_u(s_wl + s * WBUF, LDV, 16 * ks, wc0 + 32 * cb, lane));
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          acc[rb][cb] = mma32b(a[rb], bh_, acc[rb][cb]);
          acc[rb][cb] = mma32b(a[rb], bl_, acc[rb][cb]);
        }
      }
    }
  };

  auto iter = [&](auto par, int gi) {
    constexpr int P = decltype(par)::value;
    constexpr int Qs = 1 - P;
    if (n_pend) finish_n(p.dn_states + ((size_t)bh * Nc + (c_end - 1 - gi / BPC)) * DK);
    mma_blk(std::integral_constant<int, P>{}, gi);
    if (gi + 1 < NBLK) stage_blk(std::integral_constant<int, Qs>{}, gi + 1);
    if (gi + 3 < NBLK) load_blk(std::integral_constant<int, Qs>{}, gi + 3);
    __syncthreads();
  };

  if (!SIG && n_out && tid < TK) p.dn_states[((size_t)bh * Nc + c_end - 1) * DK + kt * TK + tid] = 0.0f;
  load_blk(std::integral_constant<int, 0>{}, 0);
  if (NBLK > 1) load_blk(std::integral_constant<int, 1>{}, 1);
  stage_blk(std::integral_constant<int, 0>{}, 0);
  if (NBLK > 2) load_blk(std::integral_constant<int, 0>{}, 2);
  __syncthreads();
  for (int gi = 0; gi < NBLK; gi += 2) {
    iter(std::integral_constant<int, 0>{}, gi);
    if (gi + 1 < NBLK) iter(std::integral_constant<int, 1>{}, gi + 1);
  }
  if (p.nseg > 1) {
    // the segment's own state gradient at its first chunk, for the joins:
    // fragment-lane order (8 values a lane per 16 x 32 fragment)
    if constexpr (!SIG) {
      flush_n();
      __syncthreads();
      finish_n(p.seg_n + ((size_t)bh * p.nseg + seg) * DK);
    }
    float* sc = p.seg_C + ((size_t)bh * p.nseg + seg) * DK * DV;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int kk = (kt * TK + wr0 + 32 * rb) / 16 + half, nb = (vc0 + wc0 + 32 * cb) / 32;
          float4* d = reinterpret_cast<float4*>(sc + ((size_t)(kk * (DV / 32) + nb) * 64 + lane) * 8);
          d[0] = make_float4(acc[rb][cb][8 * half], acc[rb][cb][8 * half + 1], acc[rb][cb][8 * half + 2],
                             acc[rb][cb][8 * half + 3]);
          d[1] = make_float4(acc[rb][cb][8 * half + 4], acc[rb][cb][8 * half + 5], acc[rb][cb][8 * half + 6],
                             acc[rb][cb][8 * half + 7]);
        }
    return;
  }
  if constexpr (!SIG) {
    flush_n();
    __syncthreads();
    finish_n(p.dn0 ? p.dn0 + (size_t)bh * DK : nullptr);
  }
  if (p.dC0) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int krow = kt * TK + wr0 + 32 * rb + 8 * (r >> 2) + 4 * h2 + (r & 3);
          const int vcol = vc0 + wc0 + 32 * cb + l32;
          p.dC0[(size_t)bh * DK * DV + (size_t)krow * DV + vcol] = acc[rb][cb][r];
        }
  }
}

// ---------------------------------------------------------------------------
// Joins of the segmented state-gradient recurrence.  With the decay of chunk
// c, d_c = e^{M_c + g_c - M_{c+1}} (sig gate: e^{g_c}), the recurrence
// A_c = d_c A_{c+1} + U_c (A_Nc = 0; slot c holds A_{c+1}) splits over
// segments [c0, c1): A_c = A^loc_c + (d_c ... d_{c1-1}) A_{c1}, where A^loc
// is the segment's own run from zero.  The carry kernel walks the segments
// from the last, writes the true A_{c1} into each segment's top slot c1 - 1
// (whose own value is zero) and the initial-state gradients; the fix kernel
// then adds the decayed A_{c1} to every other slot of the segment.  Values
// are handled in pieces of one fragment lane: 8 values of the packed layout.

// decay of chunk c of head bh
template <bool SIG>
__device__ __forceinline__ float chunk_decay(const BwParams& p, int bh, int c) {
  const float g = p.gb[(size_t)bh * p.S + min((c + 1) * p.L, p.S) - 1];
  if constexpr (SIG) return expf(g);
  const float* M = p.m_states + (size_t)bh * (p.Nc + 1);
  return expf(M[c] + g - M[c + 1]);
}

// piece g (fragment g / 64, lane g % 64) of slot c of the packed gradients
__device__ __forceinline__ void g_piece_load(const BwParams& p, int bh, int c, int g, float (&x)[8]) {
  const uint16_t* P = p.G_packed + ((size_t)bh * p.Nc + c) * p.DK * p.DV * 2 + (size_t)(g >> 6) * 1024 + (g & 63) * 8;
  const uint4 h = *reinterpret_cast<const uint4*>(P), l = *reinterpret_cast<const uint4*>(P + 512);
  const uint32_t hw[4] = {h.x, h.y, h.z, h.w}, lw[4] = {l.x, l.y, l.z, l.w};
#pragma unroll
  for (int e = 0; e < 8; ++e)
    x[e] = __uint_as_float(e & 1 ? hw[e >> 1] & 0xffff0000u : hw[e >> 1] << 16) +
           __uint_as_float(e & 1 ? lw[e >> 1] & 0xffff0000u : lw[e >> 1] << 16);
}
__device__ __forceinline__ void g_piece_store(const BwParams& p, int bh, int c, int g, const float (&x)[8]) {
  uint16_t* P = p.G_packed + ((size_t)bh * p.Nc + c) * p.DK * p.DV * 2 + (size_t)(g >> 6) * 1024 + (g & 63) * 8;
  uint32_t hw[4], lw[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) split_bf16x2(x[2 * q], x[2 * q + 1], hw[q], lw[q]);
  *reinterpret_cast<uint4*>(P) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
  *reinterpret_cast<uint4*>(P + 512) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
}

template <bool SIG>
__global__ __launch_bounds__(256) void bw_dstate_carry_kernel(const BwParams p) {
  const int per = p.DK * p.DV / 8;
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (long long)p.BH * per) return;
  const int bh = (int)(gid / per), g = (int)(gid % per);
  const int Nc = p.Nc, DK = p.DK, DV = p.DV;
  const bool own_n = !SIG && g < DK;  // normaliser entry g
  float A[8], An = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) A[e] = 0.0f;
  for (int s = p.nseg - 1; s >= 0; --s) {
    const int c0 = s * p.cps, c1 = min(Nc, c0 + p.cps);
    if (s < p.nseg - 1) {
      g_piece_store(p, bh, c1 - 1, g, A);
      if (own_n) p.dn_states[((size_t)bh * Nc + c1 - 1) * DK + g] = An;
    }
    float P = 1.0f;
    for (int c = c0; c < c1; ++c) P *= chunk_decay<SIG>(p, bh, c);
    const float* sc = p.seg_C + ((size_t)bh * p.nseg + s) * DK * DV + (size_t)g * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) A[e] = sc[e] + P * A[e];
    if (own_n) An = p.seg_n[((size_t)bh * p.nseg + s) * DK + g] + P * An;
  }
  if (p.dC0) {
    const int f = g >> 6, ln = g & 63, kk = f / (DV / 32), nb = f % (DV / 32);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = 16 * kk + (e < 4 ? 0 : 8) + 4 * (ln >> 5) + (e & 3);
      p.dC0[((size_t)bh * DK + k) * DV + 32 * nb + (ln & 31)] = A[e];
    }
  }
  if (own_n && p.dn0) p.dn0[(size_t)bh * DK + g] = An;
}

// One thread per (head, segment before the last, piece): the segment's top
// slot is read once, and the decay product grows as the walk goes down.
template <bool SIG>
__global__ __launch_bounds__(256) void bw_dstate_fix_kernel(const BwParams p) {
  const int per = p.DK * p.DV / 8;
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (long long)p.BH * (p.nseg - 1) * per) return;
  const int g = (int)(gid % per);
  const long long rest = gid / per;
  const int s = (int)(rest % (p.nseg - 1)), bh = (int)(rest / (p.nseg - 1));
  const int c0 = s * p.cps, c1 = c0 + p.cps;  // segments before the last are whole
  float top[8];
  g_piece_load(p, bh, c1 - 1, g, top);
  const bool own_n = !SIG && g < p.DK;
  float* dn = own_n ? p.dn_states + (size_t)bh * p.Nc * p.DK + g : nullptr;
  const float topn = own_n ? dn[(size_t)(c1 - 1) * p.DK] : 0.0f;
  float F = 1.0f;
  for (int c = c1 - 2; c >= c0; --c) {
    F *= chunk_decay<SIG>(p, bh, c + 1);
    float x[8];
    g_piece_load(p, bh, c, g, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] += F * top[e];
    g_piece_store(p, bh, c, g, x);
    if (own_n) dn[(size_t)c * p.DK] += F * topn;
  }
}

// Staging in two halves, so that the global loads of the next tile are in
// flight while the matrix cores work on the current one: pre16 loads this
// thread's 16 values of a tile into registers, put_rows writes them to LDS
// row-major as bf16, split into hi + lo where a lo plane is given (a raw bf16
// value converts exactly).
__device__ __forceinline__ void pre16(float (&x)[16], const void* src, bool bf16, size_t row0, int D, int col0,
                                      int nrows) {
  const int r = threadIdx.x >> 2, c = (threadIdx.x & 3) * 16;
  if (r < nrows) {
    load16(src, bf16, (row0 + r) * (size_t)D + col0 + c, x);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = 0.0f;
  }
}

__device__ __forceinline__ void put_rows(uint16_t* hi, uint16_t* lo, const float (&x)[16], const float* rowscale) {
  const int r = threadIdx.x >> 2, c = (threadIdx.x & 3) * 16;
  const float sc = rowscale ? rowscale[r] : 1.0f;
  uint32_t hw[8], lw[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) split_bf16x2(x[2 * i] * sc, x[2 * i + 1] * sc, hw[i], lw[i]);
  uint4* dh = reinterpret_cast<uint4*>(hi + r * kLd16 + c);
  dh[0] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
  dh[1] = make_uint4(hw[4], hw[5], hw[6], hw[7]);
  if (lo) {
    uint4* dl = reinterpret_cast<uint4*>(lo + r * kLd16 + c);
    dl[0] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    dl[1] = make_uint4(lw[4], lw[5], lw[6], lw[7]);
  }
}

// A 64 x 64 tile of a packed chunk state (16-row steps kk0 .. kk0 + 3,
// 32-column blocks nb0, nb0 + 1; layout in device_common.h), as bf16 hi and
// lo planes for put_packed_vk.  Thread t owns fragment lanes t and t + 256: its four
// 16-byte pieces (hi, lo of each) travel in x's registers.  The planes are
// the split of the float32 state already (hi + lo is exact in float32).
__device__ __forceinline__ void pre_packed(float (&x)[16], const uint16_t* P, int DV, int kk0, int nb0) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int idx = threadIdx.x + 256 * j, f = idx >> 6, lane = idx & 63;
#pragma unroll
    for (int plane = 0; plane < 2; ++plane) {
      const uint4 u = *reinterpret_cast<const uint4*>(P + pack_frag_offset(kk0 + (f >> 1), nb0 + (f & 1), plane, DV) +
                                                      lane * 8);
      x[8 * j + 4 * plane + 0] = __uint_as_float(u.x);
      x[8 * j + 4 * plane + 1] = __uint_as_float(u.y);
      x[8 * j + 4 * plane + 2] = __uint_as_float(u.z);
      x[8 * j + 4 * plane + 3] = __uint_as_float(u.w);
    }
  }
}

// The same two halves for a source that is bf16 by construction and enters
// unsplit and unscaled: the raw bf16 pairs stay packed in 8 registers (a
// raw bf16 value is its own hi part, with a zero lo part).
__device__ __forceinline__ void pre16(uint32_t (&x)[8], const void* src, bool, size_t row0, int D, int col0,
                                      int nrows) {
  const int r = threadIdx.x >> 2, c = (threadIdx.x & 3) * 16;
  uint4 a = make_uint4(0u, 0u, 0u, 0u), b = a;
  if (r < nrows) {
    const uint4* q = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + (row0 + r) * (size_t)D + col0 + c);
    a = q[0];
    b = q[1];
  }
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

__device__ __forceinline__ void put_rows(uint16_t* hi, uint16_t*, const uint32_t (&x)[8], const float*) {
  const int r = threadIdx.x >> 2, c = (threadIdx.x & 3) * 16;
  uint4* dh = reinterpret_cast<uint4*>(hi + r * kLd16 + c);
  dh[0] = make_uint4(x[0], x[1], x[2], x[3]);
  dh[1] = make_uint4(x[4], x[5], x[6], x[7]);
}

// The tile of pre_packed as [v][k] hi and lo planes: each fragment lane's
// 8 values are two runs of 4 consecutive k at one v, one 8-byte store each.
__device__ __forceinline__ void put_packed_vk(uint16_t* hi, uint16_t* lo, const float (&x)[16]) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int idx = threadIdx.x + 256 * j, f = idx >> 6, lane = idx & 63;
    const int v = 32 * (f & 1) + (lane & 31), k = 16 * (f >> 1) + 4 * (lane >> 5);
#pragma unroll
    for (int plane = 0; plane < 2; ++plane) {
      uint16_t* dst = (plane ? lo : hi) + v * kLd16 + k;
      const float* w = x + 8 * j + 4 * plane;
      *reinterpret_cast<uint2*>(dst) = make_uint2(__float_as_uint(w[0]), __float_as_uint(w[1]));
      *reinterpret_cast<uint2*>(dst + 8) = make_uint2(__float_as_uint(w[2]), __float_as_uint(w[3]));
    }
  }
}

// The values of pre16 (row r = thread / 4, columns 16 (thread % 4) + i)
// transposed, dst[c * kLd16 + r], as bf16 hi + lo.
__device__ __forceinline__ void put_cols(uint16_t* hi, uint16_t* lo, const float (&x)[16]) {
  const int r = threadIdx.x >> 2, c = (threadIdx.x & 3) * 16;
#pragma unroll
  for (int i = 0; i < 16; i += 2) {
    uint32_t hw, lw;
    split_bf16x2(x[i], x[i + 1], hw, lw);
    hi[(c + i) * kLd16 + r] = (uint16_t)(hw & 0xffff);
    hi[(c + i + 1) * kLd16 + r] = (uint16_t)(hw >> 16);
    lo[(c + i) * kLd16 + r] = (uint16_t)(lw & 0xffff);
    lo[(c + i + 1) * kLd16 + r] = (uint16_t)(lw >> 16);
  }
}

template <int MODE, bool SIG, int NY>
__device__ __forceinline__ void tiles16_body(const BwParams& p) {
  constexpr int W = 16 * NY;
  // LDS planes of 64 x kLd16 bf16, only those the mode uses (a lo plane
  // where the operand is split), so that three workgroups fit a CU:
  // partner tile [o][x] (dk: hi, lo; dv: hi; dq reads the dS tiles instead),
  // own tile [w][x] (dq: hi, lo; else hi), output-side operand (hi, lo)
  constexpr int kPl = kT * kLd16;
  constexpr int NXP = MODE == kModeDQ ? 0 : MODE == kModeDK ? 2 : 1;
  constexpr int NWP = MODE == kModeDQ ? 2 : 1;
  __shared__ __align__(16) uint16_t s_buf[(NXP + NWP + 2) * kPl];
  uint16_t* const s_x[2] = {s_buf, s_buf + (NXP > 1 ? kPl : 0)};
  uint16_t* const s_w[2] = {s_buf + NXP * kPl, s_buf + (NXP + NWP - 1) * kPl};
  uint16_t* const s_y[2] = {s_buf + (NXP + NWP) * kPl, s_buf + (NXP + NWP + 1) * kPl};
  __shared__ RowGates g_own, g_oth;

  const int nT = p.L / kT;
  const TileIdx ti = xcd_tile();
  const int ot = ti.x % nT;
  const int rest = ti.x / nT;
  const int c = rest % p.Nc, bh = rest / p.Nc;
  const int t0 = c * p.L, Lc = min(p.L, p.S - t0);
  const int own0 = ot * kT;
  if (own0 >= Lc) return;
  const int nown = min(kT, Lc - own0);
  const size_t rb = (size_t)bh * p.S + t0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g4 = lane >> 4, l16 = lane & 15;
  const int DK = p.DK, DV = p.DV, Nc = p.Nc;
  const int DO = MODE == kModeDV ? DV : DK;
  const int y0 = ti.y * W;
  const bool hb = p.dh_bf16;

  load_rows<SIG>(g_own, p, rb, own0, Lc);
  __syncthreads();
  const int w = 16 * wave + l16;
  const bool own_ok = w < nown;
  const float ob = g_own.b[w], osrc = g_own.src[w];
  const float om = SIG ? 0.0f : g_own.m[w];
  const float odelta = SIG ? 0.0f : g_own.delta[w];
  const float gc = p.gb[rb + Lc - 1];

  float4_t acc[NY];
#pragma unroll
  for (int i = 0; i < NY; ++i) acc[i] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // the own tile's operand of a contraction chunk: dH (dq), V (dk), K (dv)
  const void* own_src = MODE == kModeDQ ? p.dH : MODE == kModeDK ? p.V : p.K;
  const bool own_bf16 = MODE == kModeDQ ? hb : true;
  const int own_D = MODE == kModeDV ? DK : DV;
  constexpr bool own_split = MODE == kModeDQ;
  // the partner tile's operand of the score contraction: V (dq), dH (dk), Q (dv)
  const void* x_src = MODE == kModeDQ ? p.V : MODE == kModeDK ? p.dH : p.Q;
  const bool x_bf16 = MODE == kModeDK ? hb : true;
  constexpr bool x_split = MODE == kModeDK, w_split = MODE == kModeDQ;
  // staging registers: packed raw bf16 for the own tile (dk, dv: V, K), the
  // partner of the scores (dv: Q) and the output side (dq, dk: K, Q)
  typedef typename std::conditional<MODE != kModeDQ, uint32_t[8], float[16]>::type OwnBuf;
  typedef typename std::conditional<MODE == kModeDV, uint32_t[8], float[16]>::type XBuf;
  typedef typename std::conditional<MODE != kModeDV, uint32_t[8], float[16]>::type YBuf;
  // dk: the scores against the diagonal partner (the own rows' tile as the
  // partner) ride on the inter-chunk loop, which stages the own tile's
  // contraction chunks anyway: each chunk's partner tile goes in at the
  // loop's second state tile, and the score products join those of that
  // step (output slices of at least two 64-column state tiles).  Not dv:
  // held to three waves, the extra accumulators spill there.
  constexpr bool FUSE = MODE == kModeDK && W >= 2 * kT;
  bool fused = false;
  float4_t scd[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) scd[i] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // ---- inter-chunk term: out^T[y][w] = sum_x A[y][x] B[w][x], over (x chunk, y chunk) pairs
  {
    bool run;
    const float* St;  // the state: rows k, columns v
    if constexpr (MODE == kModeDQ) {
      run = c > 0 || p.C0 || p.n0;
      St = p.C_states + ((size_t)bh * (Nc + 1) + c) * DK * DV;
    } else {
      run = c < Nc - 1;
      St = p.dC_states + ((size_t)bh * Nc + c) * DK * DV;
    }
    if (run) {
      constexpr int NYC = W / kT;
      fused = FUSE;
      const int nxc = own_D / kT;
      // state tile of (x chunk, y chunk), held in LDS as [v][k] in every
      // mode: dq and dk (rows y = k) read it transposed, dv (rows y = v)
      // directly; packed states (dq: C; dk, dv: G)
      const uint16_t* Pk = nullptr;
      if constexpr (MODE == kModeDQ) {
        if (p.C_packed) Pk = p.C_packed + ((size_t)bh * (Nc + 1) + c) * DK * DV * 2;
      } else {
        if (p.G_packed) Pk = p.G_packed + ((size_t)bh * Nc + c) * DK * DV * 2;
      }
      auto pre_state = [&](float (&x)[16], int xi, int yc) {
        if (Pk) {
          // the 64 x 64 tile of rows k, columns v: dq and dk take k = y,
          // v = x; dv takes k = x, v = y
          if constexpr (MODE == kModeDV) pre_packed(x, Pk, DV, xi * 4, (y0 + yc * kT) / 32);
          else pre_packed(x, Pk, DV, (y0 + yc * kT) / 16, xi * 2);
          return;
        }
        if constexpr (MODE == kModeDV) pre16(x, St, false, xi * kT, DV, y0 + yc * kT, kT);
        else pre16(x, St, false, y0 + yc * kT, DV, xi * kT, kT);
      };
      OwnBuf pw;
      XBuf px;
      float py[16];
      pre16(pw, own_src, own_bf16, rb + own0, own_D, 0, nown);
      pre_state(py, 0, 0);
      for (int xi = 0; xi < nxc; ++xi) {
#pragma unroll
        for (int yc = 0; yc < NYC; ++yc) {
        __syncthreads();
        if (yc == 0) put_rows(s_w[0], own_split ? s_w[1] : nullptr, pw, own_split && !SIG ? g_own.invz : nullptr);
        if (FUSE && yc == 1) put_rows(s_x[0], x_split ? s_x[1] : nullptr, px, x_split && !SIG ? g_own.invz : nullptr);
        if (Pk) put_packed_vk(s_y[0], s_y[1], py);
        else put_cols(s_y[0], s_y[1], py);
        __syncthreads();
        if (yc + 1 < NYC) {
          pre_state(py, xi, yc + 1);
        } else if (xi + 1 < nxc) {
          pre16(pw, own_src, own_bf16, rb + own0, own_D, (xi + 1) * kT, nown);
          pre_state(py, xi + 1, 0);
        }
        if (FUSE && yc == 0) pre16(px, x_src, x_bf16, rb + own0, own_D, xi * kT, nown);
        if (FUSE && yc == 1) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int k0 = 32 * j + 8 * g4;
            const bf16x8_t bh_ = frag16(s_w[0], w, k0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float4_t a_ = mma16b(frag16(s_x[0], 16 * i + l16, k0), bh_, scd[i]);
              if constexpr (x_split) a_ = mma16b(frag16(s_x[1], 16 * i + l16, k0), bh_, a_);
              scd[i] = a_;
            }
          }
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int k0 = 32 * j + 8 * g4;
          const bf16x8_t bh_ = frag16(s_w[0], w, k0);
          bf16x8_t bl_;
          if constexpr (own_split) bl_ = frag16(s_w[1], w, k0);
#pragma unroll
          for (int yb = 0; yb < 4; ++yb) {
            // the state tile is [v][k] in LDS: dq and dk read it transposed
            const bf16x8_t ah = MODE == kModeDV ? frag16(s_y[0], 16 * yb + l16, k0) : frag16_tr(s_y[0], k0, 4, 16 * yb);
            const bf16x8_t al = MODE == kModeDV ? frag16(s_y[1], 16 * yb + l16, k0) : frag16_tr(s_y[1], k0, 4, 16 * yb);
            float4_t a_ = acc[4 * yc + yb];
            a_ = mma16b(ah, bh_, a_);
            a_ = mma16b(al, bh_, a_);
            if constexpr (own_split) a_ = mma16b(ah, bl_, a_);
            acc[4 * yc + yb] = a_;
          }
        }
        }
      }
      if constexpr (MODE == kModeDQ) {
        float wq;
        if constexpr (SIG) wq = own_ok ? expf(ob) : 0.0f;
        else wq = own_ok ? expf(ob + p.m_states[(size_t)bh * (Nc + 1) + c] - om) : 0.0f;
        const float* nst = SIG ? nullptr : p.n_states + ((size_t)bh * (Nc + 1) + c) * DK;
#pragma unroll
        for (int yb = 0; yb < NY; ++yb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float x = acc[yb][r] * wq;
            if constexpr (!SIG) x += odelta * wq * nst[y0 + 16 * yb + 4 * g4 + r];
            acc[yb][r] = x;
          }
      } else {
        const float Mo = SIG ? 0.0f : p.m_states[(size_t)bh * (Nc + 1) + c + 1];
        const float wk = own_ok ? expf(gc - ob + osrc - Mo) : 0.0f;
        if constexpr (MODE == kModeDK) {
          const float* Nst = SIG ? nullptr : p.dn_states + ((size_t)bh * Nc + c) * DK;
          const float f = wk / p.scale;
#pragma unroll
          for (int yb = 0; yb < NY; ++yb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              float x = acc[yb][r];
              if constexpr (!SIG) x += Nst[y0 + 16 * yb + 4 * g4 + r];
              acc[yb][r] = x * f;
            }
        } else {
#pragma unroll
          for (int yb = 0; yb < NY; ++yb) acc[yb] *= wk;
        }
      }
    }
  }

  // ---- intra-chunk term
  const int lo = MODE == kModeDQ ? 0 : ot;
  const int hi = MODE == kModeDQ ? ot : (Lc - 1) / kT;
  // the partner tile's operand of the output product: K (dq), Q (dk), dH (dv)
  const void* y_src = MODE == kModeDQ ? p.K : MODE == kModeDK ? p.Q : p.dH;
  const bool y_bf16 = MODE == kModeDV ? hb : true;
  const int y_D = MODE == kModeDV ? DV : DK;
  constexpr bool y_split = MODE == kModeDV;
  // the weighted dS tiles of the chunk's (query tile, key tile) pairs: the dk
  // pass writes them, the dq pass (launched after it) reads them
  float* dS_chunk = p.dS_tiles + ((size_t)bh * Nc + c) * (size_t)(nT * (nT + 1) / 2) * kT * kT;
  for (int xt = lo; xt <= hi; ++xt) {
    const int x0 = xt * kT, nx = min(kT, Lc - x0);
    float4_t sc[4];
    if constexpr (MODE == kModeDQ) {
      // dS[own query w][partner keys 16 i + 4 g4 + 0..3], weighted and masked
      const float* t = dS_chunk + ((size_t)(ot * (ot + 1) / 2 + xt) * kT + w) * kT + 4 * g4;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 v = *reinterpret_cast<const float4*>(t + 16 * i);
        sc[i] = float4_t{v.x, v.y, v.z, v.w};
      }
    } else {
    __syncthreads();
    load_rows<SIG>(g_oth, p, rb, x0, Lc);
    if (fused && xt == ot) {
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[i] = scd[i];
    } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    const int nc = own_D / kT;  // contraction chunks (the own tile's width)
    XBuf px;
    OwnBuf pw;
    pre16(px, x_src, x_bf16, rb + x0, own_D, 0, nx);
    pre16(pw, own_src, own_bf16, rb + own0, own_D, 0, nown);
    for (int ci = 0; ci < nc; ++ci) {
      __syncthreads();
      put_rows(s_x[0], x_split ? s_x[1] : nullptr, px, x_split && !SIG ? g_oth.invz : nullptr);
      put_rows(s_w[0], w_split ? s_w[1] : nullptr, pw, w_split && !SIG ? g_own.invz : nullptr);
      __syncthreads();
      if (ci + 1 < nc) {
        pre16(px, x_src, x_bf16, rb + x0, own_D, (ci + 1) * kT, nx);
        pre16(pw, own_src, own_bf16, rb + own0, own_D, (ci + 1) * kT, nown);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int k0 = 32 * j + 8 * g4;
        const bf16x8_t bh_ = frag16(s_w[0], w, k0);
        bf16x8_t bl_;
        if constexpr (w_split) bl_ = frag16(s_w[1], w, k0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16x8_t ah = frag16(s_x[0], 16 * i + l16, k0);
          float4_t a_ = mma16b(ah, bh_, sc[i]);
          if constexpr (w_split) a_ = mma16b(ah, bl_, a_);
          if constexpr (x_split) a_ = mma16b(frag16(s_x[1], 16 * i + l16, k0), bh_, a_);
          sc[i] = a_;
        }
      }
    }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int o = 16 * i + 4 * g4 + r;
        float x = 0.0f;
        // o = query, w = key
        if (own_ok && o < nx && own0 + w <= x0 + o) {
          const float ex = g_oth.b[o] - ob + osrc - (SIG ? 0.0f : g_oth.m[o]);
          if constexpr (MODE == kModeDK) x = expf(ex) * (sc[i][r] + (SIG ? 0.0f : g_oth.delta[o]));
          else x = expf(ex) * p.scale * sc[i][r];
        }
        sc[i][r] = x;
      }
    if constexpr (MODE == kModeDK) {
      // dS[partner query o][own key w] for the dq pass
      float* t = dS_chunk + ((size_t)(xt * (xt + 1) / 2 + ot) * kT) * kT + w;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) t[(16 * i + 4 * g4 + r) * kT] = sc[i][r];
    }
    }
    // first output-side tile (loads in flight during the split below)
    YBuf py;
    pre16(py, y_src, y_bf16, rb + x0, y_D, y0, nx);
    // the weighted tile as bf16 hi + lo B fragments, one per 32 partner rows
    bf16x8_t bsh[2], bsl[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      uint32_t hw[4], lw[4];
      split_bf16x2(sc[2 * q][0], sc[2 * q][1], hw[0], lw[0]);
      split_bf16x2(sc[2 * q][2], sc[2 * q][3], hw[1], lw[1]);
      split_bf16x2(sc[2 * q + 1][0], sc[2 * q + 1][1], hw[2], lw[2]);
      split_bf16x2(sc[2 * q + 1][2], sc[2 * q + 1][3], hw[3], lw[3]);
      bsh[q] = as_bf16x8(make_uint4(hw[0], hw[1], hw[2], hw[3]));
      bsl[q] = as_bf16x8(make_uint4(lw[0], lw[1], lw[2], lw[3]));
    }
    // output product: out^T[y][w] += sum_o Y[o][y] sc[o][w]
    constexpr int NYC = W / kT;
#pragma unroll
    for (int yc = 0; yc < NYC; ++yc) {
      __syncthreads();
      // Y stays [o][y] in LDS (row stores) and is read transposed
      put_rows(s_y[0], y_split ? s_y[1] : nullptr, py, y_split && !SIG ? g_oth.invz : nullptr);
      __syncthreads();
      if (yc + 1 < NYC) pre16(py, y_src, y_bf16, rb + x0, y_D, y0 + (yc + 1) * kT, nx);
#pragma unroll
      for (int yb = 0; yb < 4; ++yb) {
        float4_t a_ = acc[4 * yc + yb];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const bf16x8_t ah = frag16_tr(s_y[0], 32 * q + 4 * g4, 16, 16 * yb);
          a_ = mma16b(ah, bsh[q], a_);
          a_ = mma16b(ah, bsl[q], a_);
          if constexpr (y_split) a_ = mma16b(frag16_tr(s_y[1], 32 * q + 4 * g4, 16, 16 * yb), bsh[q], a_);
        }
        acc[4 * yc + yb] = a_;
      }
    }
  }

  // ---- epilogue (as the float32 kernel)
  const float fin = MODE == kModeDV ? 1.0f : p.scale;
  float* out = MODE == kModeDQ ? p.dQ : MODE == kModeDK ? p.dK : p.dV;
  float dot = 0.0f;
  if (own_ok) {
    const size_t orow = rb + own0 + w;
#pragma unroll
    for (int yb = 0; yb < NY; ++yb) {
      const int y = y0 + 16 * yb + 4 * g4;
      const float4 o4 = make_float4(acc[yb][0] * fin, acc[yb][1] * fin, acc[yb][2] * fin, acc[yb][3] * fin);
      *reinterpret_cast<float4*>(out + orow * DO + y) = o4;
      if constexpr (MODE != kModeDV) {
        const uint16_t* src = static_cast<const uint16_t*>(MODE == kModeDQ ? p.Q : p.K);
        const uint2 u = *reinterpret_cast<const uint2*>(src + orow * DK + y);
        dot += __uint_as_float(u.x << 16) * o4.x + __uint_as_float(u.x & 0xffff0000u) * o4.y +
               __uint_as_float(u.y << 16) * o4.z + __uint_as_float(u.y & 0xffff0000u) * o4.w;
      }
    }
  }
  if constexpr (MODE != kModeDV) {
    dot += __shfl_xor(dot, 16, 64);
    dot += __shfl_xor(dot, 32, 64);
    if (g4 == 0 && own_ok) (MODE == kModeDQ ? p.qdq : p.kdk)[rb + own0 + w] = dot;
  }
}

// Two workgroups per CU by registers; the dq and dv passes also come in a
// variant held to three (dq fits without spills, dv spills a few registers
// in its epilogue; dk would spill its accumulators).
template <int MODE, bool SIG, int NY>
__global__ __launch_bounds__(256) void bw_tiles16_kernel(const BwParams p) {
  tiles16_body<MODE, SIG, NY>(p);
}
template <int MODE, bool SIG, int NY>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void bw_tiles16_w3_kernel(const BwParams p) {
  tiles16_body<MODE, SIG, NY>(p);
}

// ---------------------------------------------------------------------------
// Gate gradients: the reverse (suffix) sum of q.dq - k.dk over the sequence,
// in blocks of 1024 positions: first every block's total, then each block's
// own scan plus the totals of the blocks after it; dm0.
constexpr int kGateBlk = 1024;
constexpr int kDm0Slices = 32;  // partial sums of dC0 . C0 per head

// Workgroups y < nblk: the total of block y; y >= nblk (exp gate, dm0
// asked): slice y - nblk of sum(dC0 * C0), beside the block totals.
__global__ __launch_bounds__(256) void bw_gate_totals_kernel(const BwParams p, int nblk) {
  __shared__ float s_w[4];
  const int blk = blockIdx.y, bh = blockIdx.x, tid = threadIdx.x;
  float a = 0.0f;
  if (blk < nblk) {
    const size_t rb = (size_t)bh * p.S;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int pos = blk * kGateBlk + 4 * tid + e;
      if (pos < p.S) a += p.qdq[rb + pos] - p.kdk[rb + pos];
    }
  } else if (p.C0) {
    // C0 and dC0 may be the caller's, 4-byte aligned only: float loads
    const size_t n = (size_t)p.DK * p.DV, len = n / kDm0Slices;  // DK DV is a multiple of 64 * 64
    const float* dc = p.dC0 + (size_t)bh * n + (blk - nblk) * len;
    const float* c0 = p.C0 + (size_t)bh * n + (blk - nblk) * len;
#pragma unroll 4
    for (size_t i = tid; i < len; i += 256) a += dc[i] * c0[i];
  }
  a = block_reduce<false, 4>(a, s_w);
  if (tid == 0) p.gate_tot[(size_t)bh * (nblk + kDm0Slices) + blk] = a;
}

template <bool SIG>
__global__ __launch_bounds__(256) void bw_gates_kernel(const BwParams p, int nblk) {
  __shared__ float s_tot[4];
  const int blk = blockIdx.y, bh = blockIdx.x, tid = threadIdx.x;
  const float* tot = p.gate_tot + (size_t)bh * (nblk + kDm0Slices);
  if (blk == nblk) {
    // dm0: the initial stabiliser enters through C0 and n0 scaled by e^{m0}
    if constexpr (!SIG) {
      float a = p.C0 && tid < kDm0Slices ? tot[nblk + tid] : 0.0f;
      if (p.n0)
        for (int i = tid; i < p.DK; i += 256) a += p.dn0[(size_t)bh * p.DK + i] * p.n0[(size_t)bh * p.DK + i];
      a = block_reduce<false, 4>(a, s_tot);
      if (tid == 0) p.dm0[bh] = a;
    }
    return;
  }
  const size_t rb = (size_t)bh * p.S;
  float carry = 0.0f;  // the blocks after this one
  for (int b = blk + 1 + tid; b < nblk; b += 256) carry += tot[b];
  carry = block_reduce<false, 4>(carry, s_tot);
  float v[4];
  int pos[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    pos[e] = blk * kGateBlk + kGateBlk - 1 - (4 * tid + e);
    v[e] = pos[e] < p.S ? p.qdq[rb + pos[e]] - p.kdk[rb + pos[e]] : 0.0f;
  }
  block_scan4<false, 4>(v, s_tot);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (pos[e] < p.S) {
      const size_t r = rb + pos[e];
      p.d_f[r] = sigmoid_neg(p.f_pre[r]) * (v[e] + carry);
      const float kd = p.kdk[r];
      p.d_i[r] = SIG ? kd * sigmoid_neg(p.i_pre[r]) : kd;
    }
  }
}

__global__ void bw_zero_kernel(float* x, long long n) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) x[i] = 0.0f;
}

hipError_t zero(float* x, long long n, hipStream_t s) {
  if (!x || n <= 0) return hipSuccess;
  hipLaunchKernelGGL(bw_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, n);
  return hipGetLastError();
}

template <int MODE, bool SIG, int NY>
void launch_tiles_ny(const BwParams& p, dim3 grid, hipStream_t s) {
  if (!p.qkv_bf16) hipLaunchKernelGGL((bw_tiles_kernel<MODE, SIG, NY>), grid, dim3(256), 0, s, p);
  else if constexpr (MODE != kModeDK) hipLaunchKernelGGL((bw_tiles16_w3_kernel<MODE, SIG, NY>), grid, dim3(256), 0, s, p);
  else hipLaunchKernelGGL((bw_tiles16_kernel<MODE, SIG, NY>), grid, dim3(256), 0, s, p);
}

template <int MODE, bool SIG>
hipError_t launch_tiles(const BwParams& p, int W, hipStream_t s) {
  const dim3 grid((unsigned)((long long)p.BH * p.Nc * (p.L / kT)), (unsigned)((MODE == kModeDV ? p.DV : p.DK) / W));
  switch (W / 16) {
    case 4: launch_tiles_ny<MODE, SIG, 4>(p, grid, s); break;
    case 8: launch_tiles_ny<MODE, SIG, 8>(p, grid, s); break;
    case 16: launch_tiles_ny<MODE, SIG, 16>(p, grid, s); break;
    case 32: launch_tiles_ny<MODE, SIG, 32>(p, grid, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool SIG>
hipError_t launch_all(const BwParams& p0, hipStream_t s) {
  hipError_t e;
  // The row-tile state recurrence (bf16 inputs, DHV 512 or 256) leaves the
  // state gradients packed, for the dk and dv passes to stage as they are.
  BwParams p = p0;
  const bool rows_kernel = p.qkv_bf16 && (p.DV == 512 || (p.DV == 256 && p.DK % 128 == 0));
  p.G_packed = rows_kernel ? reinterpret_cast<uint16_t*>(p.dC_states) : nullptr;
  hipLaunchKernelGGL((bw_prep_kernel<SIG>), dim3((unsigned)(p.BH * p.Nc)), dim3(256), 0, s, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const dim3 gs((unsigned)p.BH, (unsigned)(p.DK / kT), (unsigned)(p.DV / kT));
  if (!rows_kernel || !p.seg_C || (!SIG && !p.seg_n) || p.cps < 1) p.nseg = 1;
  // tiles of 64 x 512, 256 x 128 (float32 dH) or 128 x 256: DHQK DHV / 32768 of them per head
  const unsigned rows = (unsigned)p.BH * (unsigned)(p.DK * p.DV / 32768) * (unsigned)p.nseg;
  if (p.qkv_bf16 && p.DV == 512 && !p.dh_bf16 && p.DK % 256 == 0)
    hipLaunchKernelGGL((bw_dstate_rows_kernel<256, 128, 32, SIG, false>), dim3(rows), dim3(512), 0, s, p);
  else if (p.qkv_bf16 && p.DV == 512 && p.dh_bf16)
    hipLaunchKernelGGL((bw_dstate_rows_kernel<64, 512, 32, SIG, true>), dim3(rows), dim3(512), 0, s, p);
  else if (p.qkv_bf16 && p.DV == 512)
    hipLaunchKernelGGL((bw_dstate_rows_kernel<64, 512, 16, SIG, false>), dim3(rows), dim3(512), 0, s, p);
  else if (p.qkv_bf16 && p.DV == 256 && p.DK % 128 == 0 && p.dh_bf16)
    hipLaunchKernelGGL((bw_dstate_rows_kernel<128, 256, 32, SIG, true>), dim3(rows), dim3(512), 0, s, p);
  else if (p.qkv_bf16 && p.DV == 256 && p.DK % 128 == 0)
    hipLaunchKernelGGL((bw_dstate_rows_kernel<128, 256, 16, SIG, false>), dim3(rows), dim3(512), 0, s, p);
  else if (p.qkv_bf16) hipLaunchKernelGGL((bw_dstate16_kernel<SIG>), gs, dim3(256), 0, s, p);
  else hipLaunchKernelGGL((bw_dstate_kernel<SIG>), gs, dim3(256), 0, s, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (p.nseg > 1) {
    const long long per = (long long)p.BH * (p.DK * p.DV / 8);
    hipLaunchKernelGGL((bw_dstate_carry_kernel<SIG>), dim3((unsigned)((per + 255) / 256)), dim3(256), 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (p.cps >= 2) {
      const long long nfix = per * (p.nseg - 1);
      hipLaunchKernelGGL((bw_dstate_fix_kernel<SIG>), dim3((unsigned)((nfix + 255) / 256)), dim3(256), 0, s, p);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  // dk first: with bf16 inputs it leaves the weighted dS tiles that dq reads
  if ((e = launch_tiles<kModeDK, SIG>(p, p.DK, s)) != hipSuccess) return e;
  if ((e = launch_tiles<kModeDQ, SIG>(p, p.DK, s)) != hipSuccess) return e;
  const int Wv = p.DV % 256 == 0 ? 256 : p.DV % 128 == 0 ? 128 : 64;
  if ((e = launch_tiles<kModeDV, SIG>(p, Wv, s)) != hipSuccess) return e;
  const int nblk = (p.S + kGateBlk - 1) / kGateBlk;
  const bool dm0 = !SIG && p.dm0;
  hipLaunchKernelGGL(bw_gate_totals_kernel, dim3((unsigned)p.BH, (unsigned)(nblk + (dm0 ? kDm0Slices : 0))),
                     dim3(256), 0, s, p, nblk);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const unsigned gy = (unsigned)nblk + (dm0 ? 1u : 0u);
  hipLaunchKernelGGL((bw_gates_kernel<SIG>), dim3((unsigned)p.BH, gy), dim3(256), 0, s, p, nblk);
  return hipGetLastError();
}

}  // namespace

int bw_dstate_segments(int BH, int DK, int DV, int Nc, bool bf16_inputs, int* cps) {
  // the row-tile recurrence: one workgroup per head and TK key rows; with
  // fewer than one per CU (256 CUs) the sequence is cut into segments
  const bool rows = bf16_inputs && (DV == 512 || (DV == 256 && DK % 128 == 0));
  const long long base = (long long)BH * DK * DV / 32768;  // tiles of 32768 entries
  if (!rows || base >= 256 || Nc < 2) {
    if (cps) *cps = Nc;
    return 1;
  }
  const long long want = (256 + base - 1) / base;
  const int c = (int)((Nc + want - 1) / want);
  if (cps) *cps = c;
  return (Nc + c - 1) / c;
}

hipError_t launch_bw(const BwParams& p, bool sig, hipStream_t stream) {
  if (p.DK % kT || p.DV % kT || p.L % kT || p.DK > 512 || p.DV > 512 || p.L > 1024) return hipErrorInvalidValue;
  if (p.S == 0) {
    // no position reads the initial state: its gradients are zero
    hipError_t e = zero(p.dC0, (long long)p.BH * p.DK * p.DV, stream);
    if (e == hipSuccess) e = zero(p.dn0, (long long)p.BH * p.DK, stream);
    if (e == hipSuccess) e = zero(p.dm0, p.BH, stream);
    return e;
  }
  return sig ? launch_all<true>(p, stream) : launch_all<false>(p, stream);
}

}  // namespace mlstm
