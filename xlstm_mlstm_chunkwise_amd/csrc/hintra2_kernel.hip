// Intra-chunk parallel stage, wide-tile version for bf16 inputs (gfx950).
//
// Same arithmetic as hintra_kernel.hip (TFLA abstract: second level of
// sequence tiling inside each chunk; mLSTM readout with the normaliser and
// the max-state), organised for the large head dimensions:
//   * one workgroup (8 waves) computes TQ rows x all DV columns of H for one
//     chunk of one head, so the score tile Q.K^T is formed once;
//   * P.V and Q.C use 32x32x16 fp16 matrix-core tiles; each wave owns a
//     64-row x (DV / (8 * 64 / TQ))-column block of H in accumulators;
//   * the chunk state C arrives packed in matrix-core fragment order (written
//     so by the wide states kernel) and is loaded straight into registers;
//   * K and V are staged in LDS row-major; V is read back transposed with
//     ds_read_b64_tr_b16 since the P.V contraction runs down its rows;
//   * the score tile is computed transposed with 16x16x32 tiles (each wave
//     16 rows), turned into P = s.S.decay, split into fp16 hi + lo planes and
//     shared through LDS as the A operand of P.V.
// Keys are taken 64 at a time.
#include "device_common.h"
#include "kernels.h"

namespace mlstm {
namespace {

constexpr int kMaxL = 1024;

template <int DK, int DV, int TQ>
struct Wide {
  static constexpr int NW = 8, NT = 512, TKV = 64;
  static constexpr int NWR = TQ / 64;      // waves along rows (64 rows each)
  static constexpr int NWC = NW / NWR;     // waves along columns
  static constexpr int WC = DV / NWC;      // columns per wave
  static constexpr int CB = WC / 32;       // 32-column blocks per wave
  static constexpr int LDK = DK + 8, LDV = DV + 8, LDP = TKV + 8;
  static constexpr int K_ELEMS = TKV * LDK;
  static constexpr int P_ELEMS = TQ * LDP;   // one plane
  static constexpr int V_ELEMS = TKV * LDV;
  static constexpr int SKB = (TQ == 128) ? 4 : 2;  // 16-key score blocks per wave
  static_assert(CB >= 1 && WC % 32 == 0, "DV too small for this tile");
  static_assert(DK % 32 == 0, "DHQK must be a multiple of 32");
};

template <int DK, int DV, int TQ, bool SIG, bool SPLIT>
__global__ __launch_bounds__(512) void hintra_wide_kernel(const HintraParams p) {
  typedef Wide<DK, DV, TQ> W;
  constexpr int NKS = DK / 32;  // 16x16x32 steps over DK

  __shared__ float s_b2[kMaxL];
  __shared__ float s_u2[kMaxL];
  __shared__ float s_red[W::NW];
  __shared__ float s_row_r2[TQ], s_row_w[TQ], s_row_m2[TQ], s_row_den[TQ], s_den2[TQ];
  __shared__ float s_n[DK];
  __shared__ __align__(16) _Float16 s_k[W::K_ELEMS];
  __shared__ __align__(16) _Float16 s_ph[W::P_ELEMS];
  __shared__ __align__(16) _Float16 s_pl[W::P_ELEMS];
  __shared__ __align__(16) _Float16 s_v[W::V_ELEMS];

  const int NQT = p.L / TQ;
  // Workgroups are dealt round-robin to the 8 XCDs; remap so that the row
  // tiles of one chunk (which read the same state, keys and values) are
  // consecutive on one XCD and share its L2.
  const int nblk = gridDim.x;
  int bid = blockIdx.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int qt = bid % NQT;
  bid /= NQT;
  const int c = bid % p.Nc;
  const int bh = bid / p.Nc;
  const int S = p.S, L = p.L, Nc = p.Nc;
  const int t0 = c * L;
  const int Lc = min(L, S - t0);
  const int row0 = qt * TQ;
  if (row0 >= Lc) return;
  const int kend = min(row0 + TQ, Lc);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, l16 = lane & 15, h2 = lane >> 5, l32 = lane & 31;
  const float scale = p.scale;

  const uint16_t* Q = static_cast<const uint16_t*>(p.Q) + ((size_t)bh * S + t0) * DK;
  const uint16_t* K = static_cast<const uint16_t*>(p.K) + ((size_t)bh * S + t0) * DK;
  const uint16_t* V = static_cast<const uint16_t*>(p.V) + ((size_t)bh * S + t0) * DV;
  const float* ig = p.i_pre + (size_t)bh * S + t0;
  const float* fg = p.f_pre + (size_t)bh * S + t0;

  // ---- gates over chunk positions [0, kend): b (inclusive cumsum of log-forget),
  // u = input term - b (log2 units), prefix max of u.
  {
    float b[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int pos = 4 * tid + e;
      b[e] = pos < kend ? log_sigmoid(fg[pos]) : 0.0f;
    }
    block_scan4<false, W::NW>(b, s_red);
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
      block_scan4<true, W::NW>(u, s_red);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int pos = 4 * tid + e;
        if (pos >= row0 && pos < kend) s_row_m2[pos - row0] = u[e];
      }
    }
    __syncthreads();
    if (tid < TQ) {
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
          s_row_r2[tid] = -mx;
          s_row_w[tid] = exp2f(M2 - mx);
          s_row_m2[tid] = b2 + mx;
        }
      } else {
        s_row_r2[tid] = 0.0f;
        s_row_w[tid] = 0.0f;
        s_row_m2[tid] = 0.0f;
      }
    }
    if constexpr (!SIG) {
      const float* nst = p.n_states + ((size_t)bh * (Nc + 1) + c) * DK;
      for (int k = tid; k < DK; k += W::NT) s_n[k] = nst[k];
    }
    __syncthreads();
  }

  // Score-tile role of this wave: 16 rows (row block sr) x SKB key blocks.
  const int sr = (TQ == 128) ? wave : (wave & 3);
  const int skb0 = (TQ == 128) ? 0 : 2 * (wave >> 2);
  const int srow = sr * 16 + l16;  // row of this lane in the transposed score tile
  // Q rows as B fragments of K.Q^T (16x16x32): Q[srow][32 ks + 8 g4 + e]
  half8_t qs[NKS];
  {
    const bool ok = row0 + srow < Lc;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      uint4 u = ok ? *reinterpret_cast<const uint4*>(Q + (size_t)(row0 + srow) * DK + 32 * ks + 8 * g4)
                   : make_uint4(0, 0, 0, 0);
      qs[ks] = bf16x8_to_f16x8(u);
    }
  }
  float den_part = 0.0f;
  if constexpr (!SIG) {
    if (skb0 == 0) {
      float d = 0.0f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
        for (int e = 0; e < 8; ++e) d += static_cast<float>(qs[ks][e]) * s_n[32 * ks + 8 * g4 + e];
      }
      den_part = d * scale * s_row_w[srow];
    }
  }

  // P.V / Q.C role: rows wr0 .. wr0+63, columns wc0 .. wc0+WC-1.
  const int wr0 = (wave / W::NWC) * 64;
  const int wc0 = (wave % W::NWC) * W::WC;
  float16_t acc[2][W::CB];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < W::CB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rb][cb][r] = 0.0f;

  // ---- inter-chunk term: acc = Q . C.  The state comes packed as matrix-core
  // B fragments (hi and lo planes) and is read straight from memory, one k step
  // ahead; the Q rows use the same contraction-slot order as the packed state.
  {
    const _Float16* Pst = reinterpret_cast<const _Float16*>(p.C_states) + ((size_t)bh * (Nc + 1) + c) * DK * DV * 2;
    constexpr int NKK = DK / 16;
    uint4 bcur[W::CB][2], bnext[W::CB][2];
    uint2 qcur[2][2], qnext[2][2];
    auto load_k = [&](int kk, uint4 (&bb)[W::CB][2], uint2 (&qq)[2][2]) {
#pragma unroll
      for (int cb = 0; cb < W::CB; ++cb) {
        const int nb = (wc0 + 32 * cb) >> 5;
        bb[cb][0] = *reinterpret_cast<const uint4*>(Pst + pack_frag_offset(kk, nb, 0, DV) + lane * 8);
        if constexpr (SPLIT) bb[cb][1] = *reinterpret_cast<const uint4*>(Pst + pack_frag_offset(kk, nb, 1, DV) + lane * 8);
      }
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int row = row0 + wr0 + 32 * rb + l32;
        const uint16_t* qp = Q + (size_t)row * DK + 16 * kk + 4 * h2;
        qq[rb][0] = row < Lc ? *reinterpret_cast<const uint2*>(qp) : make_uint2(0, 0);
        qq[rb][1] = row < Lc ? *reinterpret_cast<const uint2*>(qp + 8) : make_uint2(0, 0);
      }
    };
    load_k(0, bcur, qcur);
#pragma unroll 2
    for (int kk = 0; kk < NKK; ++kk) {
      if (kk + 1 < NKK) load_k(kk + 1, bnext, qnext);
      half8_t a[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const half4_t lo4 = bf16x4_to_f16x4(qcur[rb][0]);
        const half4_t hi4 = bf16x4_to_f16x4(qcur[rb][1]);
        a[rb][0] = lo4[0]; a[rb][1] = lo4[1]; a[rb][2] = lo4[2]; a[rb][3] = lo4[3];
        a[rb][4] = hi4[0]; a[rb][5] = hi4[1]; a[rb][6] = hi4[2]; a[rb][7] = hi4[3];
      }
#pragma unroll
      for (int cb = 0; cb < W::CB; ++cb) {
        const half8_t bh_ = __builtin_bit_cast(half8_t, bcur[cb][0]);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) acc[rb][cb] = mma32(a[rb], bh_, acc[rb][cb]);
        if constexpr (SPLIT) {
          const half8_t bl_ = __builtin_bit_cast(half8_t, bcur[cb][1]);
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) acc[rb][cb] = mma32(a[rb], bl_, acc[rb][cb]);
        }
      }
      if (kk + 1 < NKK) {
#pragma unroll
        for (int cb = 0; cb < W::CB; ++cb) {
          bcur[cb][0] = bnext[cb][0];
          bcur[cb][1] = bnext[cb][1];
        }
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          qcur[rb][0] = qnext[rb][0];
          qcur[rb][1] = qnext[rb][1];
        }
      }
    }
    // scale row by e^{b + M - m} * s
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wr0 + 32 * rb + 8 * (r >> 2) + 4 * h2 + (r & 3);
        const float w = s_row_w[row] * scale;
#pragma unroll
        for (int cb = 0; cb < W::CB; ++cb) acc[rb][cb][r] *= w;
      }
  }

  // ---- intra-chunk term over key tiles [0, kend)
  const float r2 = s_row_r2[srow];
  const int tau = row0 + srow;  // chunk row of this lane in the score tile
  const int ntiles = (kend + W::TKV - 1) / W::TKV;
  // K and V tiles (64 rows) are prefetched into registers one tile ahead.
  constexpr int KPT = W::TKV * DK / 8 / W::NT;  // 16-byte K loads per thread
  constexpr int VPT = W::TKV * DV / 8 / W::NT;  // 16-byte V loads per thread
  static_assert(W::TKV * DK / 8 % W::NT == 0 && W::TKV * DV / 8 % W::NT == 0, "tile split");
  uint4 kpre[KPT], vpre[VPT];
  auto load_kv = [&](int s0) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int idx = tid + i * W::NT;
      const int rr = idx / (DK / 8), cc = (idx % (DK / 8)) * 8;
      kpre[i] = (s0 + rr < Lc) ? *reinterpret_cast<const uint4*>(K + (size_t)(s0 + rr) * DK + cc)
                               : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int idx = tid + i * W::NT;
      const int rr = idx / (DV / 8), cc = (idx % (DV / 8)) * 8;
      vpre[i] = (s0 + rr < Lc) ? *reinterpret_cast<const uint4*>(V + (size_t)(s0 + rr) * DV + cc)
                               : make_uint4(0, 0, 0, 0);
    }
  };
  if (ntiles > 0) load_kv(0);
  for (int j = 0; j < ntiles; ++j) {
    const int s0 = j * W::TKV;
    // stage K rows (64 x DK) and V rows (64 x DV) as fp16, row-major
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int idx = tid + i * W::NT;
      const int rr = idx / (DK / 8), cc = (idx % (DK / 8)) * 8;
      *reinterpret_cast<half8_t*>(s_k + rr * W::LDK + cc) = bf16x8_to_f16x8(kpre[i]);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int idx = tid + i * W::NT;
      const int rr = idx / (DV / 8), cc = (idx % (DV / 8)) * 8;
      *reinterpret_cast<half8_t*>(s_v + rr * W::LDV + cc) = bf16x8_to_f16x8(vpre[i]);
    }
    if (j + 1 < ntiles) load_kv(s0 + W::TKV);
    __syncthreads();

    // transposed scores for 16 rows x SKB key blocks; P to LDS as hi/lo planes
#pragma unroll
    for (int kb = 0; kb < W::SKB; ++kb) {
      const int sb = skb0 + kb;
      const int key0 = s0 + 16 * sb;
      float4_t sacc = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
      const bool live = key0 <= row0 + sr * 16 + 15 && key0 < kend;  // wave-uniform
      if (live) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const half8_t a = *reinterpret_cast<const half8_t*>(s_k + (16 * sb + l16) * W::LDK + 32 * ks + 8 * g4);
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qs[ks], sacc, 0, 0, 0);
        }
      }
      half4_t ph, pl;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int sg = key0 + 4 * g4 + r;
        float val = 0.0f;
        if (live && sg <= tau && tau < kend) val = scale * sacc[r] * exp2f(r2 + s_u2[sg]);
        den_part += val;
        const _Float16 hh = static_cast<_Float16>(val);
        ph[r] = hh;
        pl[r] = static_cast<_Float16>(val - static_cast<float>(hh));
      }
      *reinterpret_cast<half4_t*>(s_ph + srow * W::LDP + 16 * sb + 4 * g4) = ph;
      if constexpr (SPLIT) *reinterpret_cast<half4_t*>(s_pl + srow * W::LDP + 16 * sb + 4 * g4) = pl;
    }
    __syncthreads();

    // acc += P . V over 16-key steps
#pragma unroll
    for (int kk = 0; kk < W::TKV / 16; ++kk) {
      const int key0 = s0 + 16 * kk;
      if (key0 > row0 + wr0 + 63 || key0 >= kend) continue;  // wave-uniform: all zero
      half8_t ah[2], al[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        ah[rb] = frag_row(s_ph, W::LDP, wr0 + 32 * rb, 16 * kk, lane);
        if constexpr (SPLIT) al[rb] = frag_row(s_pl, W::LDP, wr0 + 32 * rb, 16 * kk, lane);
      }
#pragma unroll
      for (int cb = 0; cb < W::CB; ++cb) {
        const half8_t bv = frag_tr(s_v, W::LDV, 16 * kk, wc0 + 32 * cb, lane);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          acc[rb][cb] = mma32(ah[rb], bv, acc[rb][cb]);
          if constexpr (SPLIT) acc[rb][cb] = mma32(al[rb], bv, acc[rb][cb]);
        }
      }
    }
    __syncthreads();
  }

  // ---- normaliser per row, then H
  if constexpr (!SIG) {
    den_part += __shfl_xor(den_part, 16, 64);
    den_part += __shfl_xor(den_part, 32, 64);
    if (g4 == 0) {
      if (TQ == 128 || skb0 == 0) s_row_den[srow] = den_part;
      else s_den2[srow] = den_part;
    }
    __syncthreads();
    if (TQ != 128 && tid < TQ) s_row_den[tid] += s_den2[tid];
  }
  __syncthreads();
  float* Hf = static_cast<float*>(p.H);
  uint16_t* Hb = static_cast<uint16_t*>(p.H);
  const size_t hbase = ((size_t)bh * S + t0) * DV;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wr0 + 32 * rb + 8 * (r >> 2) + 4 * h2 + (r & 3);
      const int t = row0 + row;
      if (t >= Lc) continue;
      float norm = 1.0f;
      if constexpr (!SIG) norm = fmaxf(fabsf(s_row_den[row]), exp2f(-s_row_m2[row])) + p.eps;
#pragma unroll
      for (int cb = 0; cb < W::CB; ++cb) {
        float hv = acc[rb][cb][r];
        if constexpr (!SIG) hv = hv / norm;
        const size_t off = hbase + (size_t)t * DV + wc0 + 32 * cb + l32;
        if (p.h_bf16) Hb[off] = f32_to_bf16(hv);
        else Hf[off] = hv;
      }
    }
  }
  if constexpr (!SIG) {
    if (tid < TQ && row0 + tid < Lc) {
      const size_t ro = (size_t)bh * S + t0 + row0 + tid;
      if (p.m_rows) p.m_rows[ro] = s_row_m2[tid] * kLn2;
      if (p.den_rows) p.den_rows[ro] = s_row_den[tid];
    }
  }
}

template <int DK, int DV, int TQ, bool SIG, bool SPLIT>
hipError_t launch_t(const HintraParams& p, hipStream_t stream) {
  dim3 grid((unsigned)(p.BH * p.Nc * (p.L / TQ)));
  hipLaunchKernelGGL((hintra_wide_kernel<DK, DV, TQ, SIG, SPLIT>), grid, dim3(512), 0, stream, p);
  return hipGetLastError();
}

template <int DK, int DV, bool SIG, bool SPLIT>
hipError_t launch_tq(const HintraParams& p, hipStream_t stream) {
  if (p.tile_lq == 128) return launch_t<DK, DV, 128, SIG, SPLIT>(p, stream);
  if constexpr (DV >= 256) return launch_t<DK, DV, 64, SIG, SPLIT>(p, stream);
  return hipErrorInvalidValue;
}

template <bool SIG, bool SPLIT>
hipError_t launch_shape(const HintraParams& p, hipStream_t stream) {
  if (p.DK == 256 && p.DV == 512) return launch_tq<256, 512, SIG, SPLIT>(p, stream);
  if (p.DK == 256 && p.DV == 256) return launch_tq<256, 256, SIG, SPLIT>(p, stream);
  if (p.DK == 128 && p.DV == 256) return launch_tq<128, 256, SIG, SPLIT>(p, stream);
  if (p.DK == 128 && p.DV == 512) return launch_tq<128, 512, SIG, SPLIT>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace

bool hintra_wide_supported(int DK, int DV, int L, int tile_lq, bool bf16_inputs) {
  if (!bf16_inputs || L < 64) return false;
  const bool shape = (DK == 256 && (DV == 512 || DV == 256)) || (DK == 128 && (DV == 256 || DV == 512));
  if (!shape) return false;
  if (tile_lq == 128) return L >= 128;
  return tile_lq == 64;
}

hipError_t launch_hintra_wide(const HintraParams& p, bool sig, bool split, hipStream_t stream) {
  if (sig) return split ? launch_shape<true, true>(p, stream) : launch_shape<true, false>(p, stream);
  return split ? launch_shape<false, true>(p, stream) : launch_shape<false, false>(p, stream);
}

}  // namespace mlstm
