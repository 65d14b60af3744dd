// Intra-chunk parallel stage of the chunkwise mLSTM forward pass (gfx950).
//
// TFLA's second level of tiling (TFLA abstract: sequence parallelism inside
// each chunk, so chunks can be large): every workgroup computes one
// TQ-row x 64-column tile of H for one chunk of one head and walks the key
// tiles of that chunk at or below the diagonal.  For chunk-local row tau and
// key sigma <= tau, with b the inclusive in-chunk sum of log-forget gates and
// (C, n, M) the stabilised state entering the chunk:
//   exp gate:  m_tau   = b_tau + max(M, max_{sigma<=tau} (i_sigma - b_sigma))
//              P       = s (q_tau . k_sigma) e^{b_tau - b_sigma + i_sigma - m_tau}
//              num     = sum_sigma P v_sigma + e^{b_tau + M - m_tau} s C^T q_tau
//              den     = sum_sigma P         + e^{b_tau + M - m_tau} s n . q_tau
//              h_tau   = num / (max(|den|, e^{-m_tau}) + eps)
//   sig gate:  P       = s (q_tau . k_sigma) e^{b_tau - b_sigma + log sigmoid(i_sigma)}
//              h_tau   = sum_sigma P v_sigma + e^{b_tau} s C^T q_tau
// The row max-state is a prefix max known before the key loop, so no running
// rescale of the accumulators is needed.  All exponentials are taken in base
// 2 on log2-scaled gate sums.
//
// Work split: TQ/16 waves; wave w owns rows 16w .. 16w+15 of the tile.  Keys
// are taken TKV at a time (TQ, TKV in {64, 128}).  H columns are split into
// 64-wide tiles across the grid.  Its Q rows
// sit in registers as matrix-core fragments for the whole kernel and serve
// both as the A operand of Q.C and as the B operand of K.Q^T.  The score tile
// is computed transposed (keys x rows) so that each lane ends up holding four
// consecutive keys of one row: two such 16 x 16 tiles form the A fragment of
// the P.V product directly (the contraction slots are permuted consistently
// on the V side), with no trip through LDS.
#include "device_common.h"
#include "tile_order.h"
#include "kernels.h"

namespace mlstm {
namespace {

constexpr int kTV = 64;     // H columns per workgroup
constexpr int kMaxL = 1024;

template <typename TIn, bool SIG, bool SPLIT, int DK, int kTQ, int kTKV>
__global__ __launch_bounds__(kTQ * 4) void hintra_kernel(const HintraParams p) {
  constexpr int NW = kTQ / 16;      // waves
  constexpr int NT = 64 * NW;       // threads
  typedef Ops<TIn> O;
  typedef typename O::lds_t lds_t;
  typedef typename O::frag frag;
  constexpr int kPad = sizeof(lds_t) == 2 ? 8 : 4;
  constexpr int NKS = DK / 32;

  __shared__ float s_b2[kMaxL];   // log2e * inclusive log-forget sum
  __shared__ float s_u2[kMaxL];   // log2e * (input gate term - b)
  __shared__ float s_red[NW];
  __shared__ float s_row_r2[kTQ], s_row_w[kTQ], s_row_m2[kTQ], s_row_den[kTQ];
  __shared__ float s_n[DK];
  __shared__ __align__(16) lds_t s_k[kTKV][DK + kPad];     // key rows [sigma][k]
  __shared__ __align__(16) lds_t s_vt[kTV][kTKV + kPad];   // values [v][sigma]
  __shared__ __align__(16) float s_ct[kTV][64 + 4];        // state slice [v][k]

  const int NQT = p.L > kTQ ? p.L / kTQ : 1;  // chunks below one tile: one tile
  const TileIdx ti = xcd_tile();
  int bid = ti.x;
  const int qt = bid % NQT;
  bid /= NQT;
  const int c = bid % p.Nc;
  const int bh = bid / p.Nc;
  const int vt = ti.y;
  const int S = p.S, DV = p.DV, L = p.L, Nc = p.Nc;
  const int t0 = c * L;
  const int Lc = min(L, S - t0);
  const int row0 = qt * kTQ;
  if (row0 >= Lc) return;
  const int kend = min(row0 + kTQ, Lc);  // keys [0, kend) are needed

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, l16 = lane & 15;
  const float scale = p.scale;

  const TIn* Q = static_cast<const TIn*>(p.Q) + ((size_t)bh * S + t0) * DK;
  const TIn* K = static_cast<const TIn*>(p.K) + ((size_t)bh * S + t0) * DK;
  const TIn* V = static_cast<const TIn*>(p.V) + ((size_t)bh * S + t0) * DV + vt * kTV;
  const float* ig = p.i_pre + (size_t)bh * S + t0;
  const float* fg = p.f_pre + (size_t)bh * S + t0;

  // ---- gates over chunk positions [0, kend)
  {
    float b[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int pos = 4 * tid + e;
      b[e] = pos < kend ? log_sigmoid(fg[pos]) : 0.0f;
    }
    block_scan4<false, NW>(b, s_red);
    float u[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int pos = 4 * tid + e;
      if (pos < kend) {
        const float it = ig[pos];
        u[e] = ((SIG ? log_sigmoid(it) : it) - b[e]) * kLog2e;
        s_b2[pos] = b[e] * kLog2e;
        s_u2[pos] = u[e];
      } else {
        u[e] = -INFINITY;
      }
    }
    if constexpr (!SIG) {
      block_scan4<true, NW>(u, s_red);  // prefix max of u
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int pos = 4 * tid + e;
        if (pos >= row0 && pos < kend) s_row_m2[pos - row0] = u[e];  // temporarily: prefix max
      }
    }
    __syncthreads();
    if (tid < kTQ) {
      const int pos = row0 + tid;
      if (pos < kend) {
        const float b2 = s_b2[pos];
        if constexpr (SIG) {
          s_row_r2[tid] = b2;
          s_row_w[tid] = exp2f(b2);
          s_row_m2[tid] = 0.0f;
        } else {
          const float M2 = p.m_states[(size_t)bh * (Nc + 1) + c] * kLog2e;
          const float mx = fmaxf(M2, s_row_m2[tid]);
          s_row_r2[tid] = -mx;             // b - m, in log2 units
          s_row_w[tid] = exp2f(M2 - mx);   // e^{b + M - m}
          s_row_m2[tid] = b2 + mx;         // m, in log2 units
        }
      } else {
        s_row_r2[tid] = 0.0f;
        s_row_w[tid] = 0.0f;
        s_row_m2[tid] = 0.0f;
      }
    }
    if constexpr (!SIG) {
      const float* nst = p.n_states + ((size_t)bh * (Nc + 1) + c) * DK;
      for (int k = tid; k < DK; k += NT) s_n[k] = nst[k];
    }
    __syncthreads();
  }

  // ---- this lane's Q row (A layout: row l16 of the wave, slots 8*g4+e)
  const int qrow = row0 + 16 * wave + l16;
  frag qf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    float x[8];
    if (qrow < Lc) {
      O::load8(Q + (size_t)qrow * DK + 32 * ks + 8 * g4, x);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.0f;
    }
    qf[ks] = O::round(x);
  }

  // ---- inter-chunk term: acc = Q . C (then scaled per row)
  float4_t acc[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) acc[nb] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const float* Cst = p.C_states + ((size_t)bh * (Nc + 1) + c) * DK * DV + vt * kTV;
  for (int kb = 0; kb < DK / 64; ++kb) {
    for (int idx = tid; idx < 64 * 16; idx += NT) {
      const int kk = idx >> 4, seg = idx & 15;
      const float4 x = *reinterpret_cast<const float4*>(Cst + (size_t)(kb * 64 + kk) * DV + seg * 4);
      s_ct[seg * 4 + 0][kk] = x.x;
      s_ct[seg * 4 + 1][kk] = x.y;
      s_ct[seg * 4 + 2][kk] = x.z;
      s_ct[seg * 4 + 3][kk] = x.w;
    }
    __syncthreads();
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        float xb[8];
        const float4 lo4 = *reinterpret_cast<const float4*>(&s_ct[16 * nb + l16][32 * ks2 + 8 * g4]);
        const float4 hi4 = *reinterpret_cast<const float4*>(&s_ct[16 * nb + l16][32 * ks2 + 8 * g4 + 4]);
        xb[0] = lo4.x; xb[1] = lo4.y; xb[2] = lo4.z; xb[3] = lo4.w;
        xb[4] = hi4.x; xb[5] = hi4.y; xb[6] = hi4.z; xb[7] = hi4.w;
        acc[nb] = mma_computed_b<TIn, SPLIT>(qf[kb * 2 + ks2], xb, acc[nb]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float w = s_row_w[16 * wave + 4 * g4 + r] * scale;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[nb][r] *= w;
  }
  float den_part = 0.0f;
  if constexpr (!SIG) {
    float d = 0.0f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float qv;
        if constexpr (sizeof(lds_t) == 2) {
          qv = static_cast<float>(qf[ks][e]);
        } else {
          qv = reinterpret_cast<const f32frag&>(qf[ks]).v[e];
        }
        d += qv * s_n[32 * ks + 8 * g4 + e];
      }
    }
    den_part = d * scale * s_row_w[16 * wave + l16];
  }

  // ---- intra-chunk term over key tiles [0, kend)
  const int tau = row0 + 16 * wave + l16;  // this lane's row in the score tiles
  const float r2 = s_row_r2[16 * wave + l16];
  const int ntiles = (kend + kTKV - 1) / kTKV;
  for (int j = 0; j < ntiles; ++j) {
    const int s0 = j * kTKV;
    for (int idx = tid; idx < kTKV * (DK / 8); idx += NT) {
      const int sg = idx / (DK / 8), seg = idx % (DK / 8);
      float x[8];
      if (s0 + sg < Lc) {
        O::load8(K + (size_t)(s0 + sg) * DK + seg * 8, x);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = 0.0f;
      }
      O::store8(&s_k[sg][seg * 8], x);
    }
    for (int idx = tid; idx < kTKV * 8; idx += NT) {
      const int sg = idx >> 3, seg = idx & 7;
      float x[8];
      if (s0 + sg < Lc) {
        O::load8(V + (size_t)(s0 + sg) * DV + seg * 8, x);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = 0.0f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) s_vt[seg * 8 + e][sg] = O::to_lds(x[e]);
    }
    __syncthreads();

    // transposed scores: sacc[mb][r] = q_tau . k_sigma, sigma = s0 + 16mb + 4g4 + r
    float pv[kTKV / 16][4];
#pragma unroll
    for (int mb = 0; mb < kTKV / 16; ++mb) {
      float4_t sacc = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const frag a = O::lds_frag(&s_k[16 * mb + l16][32 * ks + 8 * g4]);
        sacc = O::mma(a, qf[ks], sacc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int sg = s0 + 16 * mb + 4 * g4 + r;
        float val = 0.0f;
        if (sg <= tau && tau < kend) val = scale * sacc[r] * exp2f(r2 + s_u2[sg]);
        pv[mb][r] = val;
        den_part += val;
      }
    }
    // acc += P . V ; contraction slot (g4, e) <-> key s0 + 32p + (e < 4 ? 4g4+e : 16+4g4+e-4)
#pragma unroll
    for (int pp = 0; pp < kTKV / 32; ++pp) {
      float xa[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xa[e] = pv[2 * pp][e];
        xa[4 + e] = pv[2 * pp + 1][e];
      }
      frag ahi, alo;
      if constexpr (SPLIT && O::kSplitCapable) {
        O::split(xa, ahi, alo);
      } else {
        ahi = O::round(xa);
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const frag bv = O::lds_frag2(&s_vt[16 * nb + l16][32 * pp + 4 * g4],
                                     &s_vt[16 * nb + l16][32 * pp + 16 + 4 * g4]);
        acc[nb] = O::mma(ahi, bv, acc[nb]);
        if constexpr (SPLIT && O::kSplitCapable) acc[nb] = O::mma(alo, bv, acc[nb]);
      }
    }
    __syncthreads();
  }

  // ---- normalise and store
  if constexpr (!SIG) {
    den_part += __shfl_xor(den_part, 16, 64);
    den_part += __shfl_xor(den_part, 32, 64);
    if (g4 == 0) s_row_den[16 * wave + l16] = den_part;
  }
  __syncthreads();
  float* Hf = static_cast<float*>(p.H);
  uint16_t* Hb = static_cast<uint16_t*>(p.H);
  const size_t hbase = ((size_t)bh * S + t0) * DV + vt * kTV;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 16 * wave + 4 * g4 + r;
    const int t = row0 + row;
    if (t >= Lc) continue;
    float norm = 1.0f;
    if constexpr (!SIG) norm = fmaxf(fabsf(s_row_den[row]), exp2f(-s_row_m2[row])) + p.eps;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      float h = acc[nb][r];
      if constexpr (!SIG) h = h / norm;
      const size_t off = hbase + (size_t)t * DV + 16 * nb + l16;
      if (p.h_bf16) {
        Hb[off] = f32_to_bf16(h);
      } else {
        Hf[off] = h;
      }
    }
  }
  if constexpr (!SIG) {
    if (vt == 0 && tid < kTQ && row0 + tid < Lc) {
      const size_t ro = (size_t)bh * S + t0 + row0 + tid;
      if (p.m_rows) p.m_rows[ro] = s_row_m2[tid] * kLn2;
      if (p.den_rows) p.den_rows[ro] = s_row_den[tid];
    }
  }
}

template <typename TIn, bool SIG, bool SPLIT, int DK, int TQ, int TKV>
hipError_t launch_t(const HintraParams& p, hipStream_t stream) {
  const int NQT = p.L > TQ ? p.L / TQ : 1;
  dim3 grid((unsigned)(p.BH * p.Nc * NQT), p.DV / kTV);
  hipLaunchKernelGGL((hintra_kernel<TIn, SIG, SPLIT, DK, TQ, TKV>), grid, dim3(TQ * 4), 0, stream, p);
  return hipGetLastError();
}

template <typename TIn, bool SIG, bool SPLIT, int DK>
hipError_t launch_tiles(const HintraParams& p, hipStream_t stream) {
  const int tq = p.tile_lq, tkv = p.tile_lkv;
  if (tq == 64 && tkv == 64) return launch_t<TIn, SIG, SPLIT, DK, 64, 64>(p, stream);
  if (tq == 128 && tkv == 64) return launch_t<TIn, SIG, SPLIT, DK, 128, 64>(p, stream);
  // A 128-key tile keeps 128 key rows of DK elements in LDS.
  if constexpr (DK * sizeof(typename Ops<TIn>::lds_t) <= 512) {
    if (tq == 128 && tkv == 128) return launch_t<TIn, SIG, SPLIT, DK, 128, 128>(p, stream);
    if (tq == 64 && tkv == 128) return launch_t<TIn, SIG, SPLIT, DK, 64, 128>(p, stream);
  }
  return hipErrorInvalidValue;
}

template <typename TIn, bool SIG, bool SPLIT>
hipError_t launch_dk(const HintraParams& p, hipStream_t stream) {
  switch (p.DK) {
    case 64: return launch_tiles<TIn, SIG, SPLIT, 64>(p, stream);
    case 128: return launch_tiles<TIn, SIG, SPLIT, 128>(p, stream);
    case 256: return launch_tiles<TIn, SIG, SPLIT, 256>(p, stream);
    default: break;
  }
  if constexpr (sizeof(typename Ops<TIn>::lds_t) == 2) {
    // 128-key tiles of 512-wide keys do not fit in LDS; validation keeps
    // tile_lkv at 64 for DHQK = 512.
    if (p.DK == 512) return launch_t<TIn, SIG, SPLIT, 512, 64, 64>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_hintra(const HintraParams& p, bool bf16_inputs, bool sig, bool split, hipStream_t stream) {
  if (!bf16_inputs) return sig ? launch_dk<float, true, false>(p, stream) : launch_dk<float, false, false>(p, stream);
  if (sig) return split ? launch_dk<bf16_t, true, true>(p, stream) : launch_dk<bf16_t, true, false>(p, stream);
  return split ? launch_dk<bf16_t, false, true>(p, stream) : launch_dk<bf16_t, false, false>(p, stream);
}

}  // namespace mlstm
