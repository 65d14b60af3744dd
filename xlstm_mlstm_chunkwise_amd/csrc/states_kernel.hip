// Inter-chunk recurrence of the chunkwise mLSTM forward pass (gfx950).
//
// For every head the kernel walks the chunks in order and materialises the
// stabilised state (C, n, M) entering each chunk, plus the final state.  The
// per-chunk update is the chunkwise form of the mLSTM recurrence (TFLA
// abstract: chunkwise-parallel linear RNN, states carried between chunks):
// with b the inclusive in-chunk sum of log-forget gates and g = b at the
// chunk's last step,
//   exp gate:  a_t   = g - b_t + i_t,      M' = max(g + M, max_t a_t)
//              C'    = e^{g + M - M'} C + sum_t e^{a_t - M'} k_t v_t^T
//              n'    = e^{g + M - M'} n + sum_t e^{a_t - M'} k_t
//   sig gate:  C'    = e^{g} C + sum_t e^{g - b_t + log sigmoid(i_t)} k_t v_t^T
//
// Work split: one workgroup (4 waves) owns a 64 x 64 tile of C for one head
// and keeps it in matrix-core accumulators across the whole sequence; wave w
// holds rows 16w .. 16w+15 of the tile.  The sum over t is a 64 x Lc x 64
// product per chunk with the time axis as contraction axis; keys (scaled by
// their gate weight) and values are staged through LDS transposed so each
// lane reads its eight contraction values contiguously.
#include "device_common.h"
#include "kernels.h"

namespace mlstm {
namespace {

constexpr int kTT = 64;     // time steps per LDS stage
constexpr int kTile = 64;   // C tile edge
constexpr int kMaxL = 1024; // largest chunk

template <typename TIn, bool SIG, bool SPLIT>
__global__ __launch_bounds__(256) void states_kernel(const StatesParams p) {
  typedef Ops<TIn> O;
  typedef typename O::lds_t lds_t;
  typedef typename O::frag frag;
  constexpr int kVPad = sizeof(lds_t) == 2 ? 8 : 4;

  __shared__ float s_w[kMaxL];                       // key weights of the chunk
  __shared__ float s_red[8];
  __shared__ float s_g;
  __shared__ __align__(16) float s_kw[kTile][kTT + 4];   // gated keys [k][t]
  __shared__ __align__(16) lds_t s_vt[kTile][kTT + kVPad];  // values [v][t]

  const int bh = blockIdx.x, kt = blockIdx.y, vt = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, l16 = lane & 15;
  const int S = p.S, DK = p.DK, DV = p.DV, L = p.L, Nc = p.Nc;
  const TIn* K = static_cast<const TIn*>(p.K) + (size_t)bh * S * DK;
  const TIn* V = static_cast<const TIn*>(p.V) + (size_t)bh * S * DV;
  const float* ig = p.i_pre + (size_t)bh * S;
  const float* fg = p.f_pre + (size_t)bh * S;
  const bool own_n = !SIG && vt == 0;

  float4_t acc[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int krow = kt * kTile + 16 * wave + 4 * g4 + r;
      const int vcol = vt * kTile + 16 * nb + l16;
      acc[nb][r] = p.C0 ? p.C0[(size_t)bh * DK * DV + (size_t)krow * DV + vcol] : 0.0f;
    }
  }
  float nreg = 0.0f;
  if (own_n && tid < kTile && p.n0) nreg = p.n0[(size_t)bh * DK + kt * kTile + tid];
  float M = 0.0f;
  if (!SIG && p.m0) M = p.m0[bh];

  for (int c = 0; c <= Nc; ++c) {
    // State entering chunk c (c == Nc: the final state).
    {
      float* Cst = p.C_states + ((size_t)bh * (Nc + 1) + c) * DK * DV;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int krow = kt * kTile + 16 * wave + 4 * g4 + r;
          const int vcol = vt * kTile + 16 * nb + l16;
          Cst[(size_t)krow * DV + vcol] = acc[nb][r];
        }
      }
      if (own_n && tid < kTile) p.n_states[((size_t)bh * (Nc + 1) + c) * DK + kt * kTile + tid] = nreg;
      if (!SIG && kt == 0 && vt == 0 && tid == 0) p.m_states[(size_t)bh * (Nc + 1) + c] = M;
    }
    if (c == Nc) break;

    const int t0 = c * L;
    const int Lc = min(L, S - t0);
    // Gates: thread t handles chunk positions 4t .. 4t+3.
    float b[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int pos = 4 * tid + e;
      b[e] = pos < Lc ? log_sigmoid(fg[t0 + pos]) : 0.0f;
    }
    block_scan4<false, 4>(b, s_red);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (4 * tid + e == Lc - 1) s_g = b[e];
    __syncthreads();
    const float gsum = s_g;
    float a[4];
    float amax = -INFINITY;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int pos = 4 * tid + e;
      if (pos < Lc) {
        const float it = ig[t0 + pos];
        a[e] = gsum - b[e] + (SIG ? log_sigmoid(it) : it);
        amax = fmaxf(amax, a[e]);
      } else {
        a[e] = -INFINITY;
      }
    }
    float decay;
    if constexpr (SIG) {
      decay = expf(gsum);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int pos = 4 * tid + e;
        if (pos < kMaxL) s_w[pos] = pos < Lc ? expf(a[e]) : 0.0f;
      }
    } else {
      amax = block_reduce<true, 4>(amax, s_red);
      const float Mnew = fmaxf(gsum + M, amax);
      decay = expf(gsum + M - Mnew);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int pos = 4 * tid + e;
        if (pos < kMaxL) s_w[pos] = pos < Lc ? expf(a[e] - Mnew) : 0.0f;
      }
      M = Mnew;
    }
    __syncthreads();
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[nb] *= decay;
    nreg *= decay;

    const TIn* Kc = K + (size_t)t0 * DK + kt * kTile;
    const TIn* Vc = V + (size_t)t0 * DV + vt * kTile;
    for (int tb = 0; tb < Lc; tb += kTT) {
      // Stage gated keys (float) and values (operand type), both transposed.
      for (int idx = tid; idx < kTT * 8; idx += 256) {
        const int t = idx >> 3, seg = idx & 7;
        float x[8];
        if (tb + t < Lc) {
          O::load8(Kc + (size_t)(tb + t) * DK + seg * 8, x);
          const float w = s_w[tb + t];
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] *= w;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = 0.0f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) s_kw[seg * 8 + e][t] = x[e];
      }
      for (int idx = tid; idx < kTT * 8; idx += 256) {
        const int t = idx >> 3, seg = idx & 7;
        float x[8];
        if (tb + t < Lc) {
          O::load8(Vc + (size_t)(tb + t) * DV + seg * 8, x);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = 0.0f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) s_vt[seg * 8 + e][t] = O::to_lds(x[e]);
      }
      __syncthreads();
      if (own_n && tid < kTile) {
        float sacc = 0.0f;
        for (int t = 0; t < kTT; ++t) sacc += s_kw[tid][t];
        nreg += sacc;
      }
#pragma unroll
      for (int ks = 0; ks < kTT / 32; ++ks) {
        float xa[8];
        const float4 lo4 = *reinterpret_cast<const float4*>(&s_kw[16 * wave + l16][32 * ks + 8 * g4]);
        const float4 hi4 = *reinterpret_cast<const float4*>(&s_kw[16 * wave + l16][32 * ks + 8 * g4 + 4]);
        xa[0] = lo4.x; xa[1] = lo4.y; xa[2] = lo4.z; xa[3] = lo4.w;
        xa[4] = hi4.x; xa[5] = hi4.y; xa[6] = hi4.z; xa[7] = hi4.w;
        frag ahi, alo;
        if constexpr (SPLIT && O::kSplitCapable) {
          O::split(xa, ahi, alo);
        } else {
          ahi = O::round(xa);
        }
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const frag bv = O::lds_frag(&s_vt[16 * nb + l16][32 * ks + 8 * g4]);
          acc[nb] = O::mma(ahi, bv, acc[nb]);
          if constexpr (SPLIT && O::kSplitCapable) acc[nb] = O::mma(alo, bv, acc[nb]);
        }
      }
      __syncthreads();
    }
  }

  if (p.C_out) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int krow = kt * kTile + 16 * wave + 4 * g4 + r;
        const int vcol = vt * kTile + 16 * nb + l16;
        p.C_out[(size_t)bh * DK * DV + (size_t)krow * DV + vcol] = acc[nb][r];
      }
    }
  }
  if (own_n && p.n_out && tid < kTile) p.n_out[(size_t)bh * DK + kt * kTile + tid] = nreg;
  if (!SIG && p.m_out && kt == 0 && vt == 0 && tid == 0) p.m_out[bh] = M;
}

template <typename TIn, bool SIG, bool SPLIT>
hipError_t launch_t(const StatesParams& p, hipStream_t stream) {
  dim3 grid(p.BH, p.DK / kTile, p.DV / kTile);
  hipLaunchKernelGGL((states_kernel<TIn, SIG, SPLIT>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_states(const StatesParams& p, bool bf16_inputs, bool sig, bool split, hipStream_t stream) {
  if (!bf16_inputs) return sig ? launch_t<float, true, false>(p, stream) : launch_t<float, false, false>(p, stream);
  if (sig) return split ? launch_t<bf16_t, true, true>(p, stream) : launch_t<bf16_t, true, false>(p, stream);
  return split ? launch_t<bf16_t, false, true>(p, stream) : launch_t<bf16_t, false, false>(p, stream);
}

}  // namespace mlstm
