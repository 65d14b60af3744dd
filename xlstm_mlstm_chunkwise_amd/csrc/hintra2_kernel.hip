// Intra-chunk parallel stage, wide-tile version for bf16 inputs (gfx950).
//
// Same arithmetic as hintra_kernel.hip (TFLA abstract: second level of
// sequence tiling inside each chunk; mLSTM readout with the normaliser and
// the max-state), organised for the large head dimensions:
//   * one workgroup (8 waves) computes TQ rows x TV columns of H for one chunk
//     of one head (TV = DV, or DV / 2 with 128-row tiles, which halves how
//     often the chunk state is read at the cost of forming the score tile
//     twice);
//   * all products run on bf16 matrix cores: Q, K, V enter unchanged, and each
//     operand computed in float32 (P = s.S.decay, the chunk state C) is carried
//     as a bf16 hi + lo pair, two MFMA passes;
//   * P.V and Q.C use 32x32x16 tiles; each wave owns a 64-row x
//     (TV / (8 * 64 / TQ))-column block of H in accumulators;
//   * the chunk state C arrives packed in matrix-core fragment order (written
//     so by the wide states kernel) and is loaded straight into registers,
//     several k steps ahead;
//   * K and V are staged in LDS row-major; V is read back transposed with
//     ds_read_b64_tr_b16 since the P.V contraction runs down its rows;
//   * the score tile is computed transposed with 16x16x32 tiles (each wave
//     16 rows), turned into P, and shared through LDS as hi and lo planes.
// Keys are taken 64 at a time.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "pair_store.h"

namespace mlstm {
namespace {

constexpr int kMaxL = 1024;

template <int DK, int TV, int TQ>
struct Wide {
  static constexpr int NW = 8, NT = 512, TKV = 64;
  static constexpr int NWR = TQ / 64;      // waves along rows (64 rows each)
  static constexpr int NWC = NW / NWR;     // waves along columns
  static constexpr int WC = TV / NWC;      // columns per wave
  static constexpr int CB = WC / 32;       // 32-column blocks per wave
  // Row strides (elements).  K and P are read along rows with 16-byte reads
  // (16 lanes, 16 rows: a stride of 4 banks mod 64 keeps them apart).  V is
  // read down its rows with ds_read_b64_tr_b16, where each half-wave takes
  // 4 rows x 64 bytes: a stride of 16 banks mod 64 keeps the rows apart.
  static constexpr int LDK = DK + 8, LDV = TV + 32, LDP = TKV + 8, LDQ = DK + 8;
  static constexpr int K_ELEMS = TKV * LDK;
  static constexpr int P_ELEMS = TQ * LDP;   // one plane
  static constexpr int V_ELEMS = TKV * LDV;
  static constexpr int Q_ELEMS = TQ * LDQ;   // shares the K/P/V space before the key loop
  static constexpr int BUF_ELEMS = (K_ELEMS + 2 * P_ELEMS + V_ELEMS) > Q_ELEMS ? (K_ELEMS + 2 * P_ELEMS + V_ELEMS)
                                                                                 : Q_ELEMS;
  static constexpr int SKB = (TQ == 128) ? 4 : 2;  // 16-key score blocks per wave
  static_assert(CB >= 1 && WC % 32 == 0, "TV too small for this tile");
  static_assert(DK % 32 == 0, "DHQK must be a multiple of 32");
};

// CODES: the chunk states arrive as int16 codes with one power-of-two scale
// per fragment (HintraParams::C_scales); each lane turns its eight codes of a
// fragment into the bf16 hi + lo pair of code * scale, which is exact (a
// code has at most 15 significant bits), right before the products.
template <int DK, int DV, int TQ, int TV, bool SIG, bool SPLIT, bool DELTA = false, bool CODES = false>
__global__ __launch_bounds__(512) void hintra_wide_kernel(const HintraParams p) {
  static_assert(!DELTA || (!SIG && TV == DV), "the row terms of the gradient need whole rows (exp gate)");
  static_assert(!CODES || (SPLIT && !DELTA), "int16-coded states feed the split forward");
  typedef Wide<DK, TV, TQ> W;
  constexpr int NVT = DV / TV;
  constexpr int NKS = DK / 32;  // 16x16x32 steps over DK
  constexpr int NKK = DK / 16;  // 32x32x16 steps over DK

  __shared__ __align__(16) float s_u2[kMaxL];
  __shared__ float s_row_r2[TQ], s_row_w[TQ], s_row_m2[TQ], s_row_den[TQ];
  __shared__ __align__(16) float s_den2[TQ];
  __shared__ float s_n[DK];
  __shared__ __align__(16) uint16_t s_buf[W::BUF_ELEMS];
  uint16_t* const s_k = s_buf;
  uint16_t* const s_ph = s_buf + W::K_ELEMS;
  uint16_t* const s_pl = s_ph + W::P_ELEMS;
  uint16_t* const s_v = s_pl + W::P_ELEMS;
  uint16_t* const s_q = s_buf;  // the Q tile, before the key loop

  const int S = p.S, L = p.L;
  const int NQT = L / TQ;
  const float scale = p.scale;
  // chunks [c_lo, c_lo + NCB) of this launch; the state entering chunk c sits
  // at slot c - c_lo of the head's SL slots
  const int c_lo = p.c_lo;
  const int NCB = (p.c_hi < 0 ? p.Nc : p.c_hi) - c_lo;
  const int SL = p.slots ? p.slots : p.Nc + 1;
  // Per-lane and per-wave roles.  They are re-derived at the top of every
  // tile from a laundered thread index, so the compiler rebuilds the offsets
  // that depend on them instead of keeping them live across the tile loop.
  int tid, lane, wave, g4, l16, h2, l32;
  int wr0, wc0;    // P.V / Q.C role: rows wr0 .. wr0+63, columns wc0 .. wc0+WC-1
  int sr, skb0;    // score-tile role: 16 rows (row block sr) x SKB key blocks
  int srow;        // row of this lane in the transposed score tile
  auto set_roles = [&]() {
    int t = (int)threadIdx.x;
    asm volatile("" : "+v"(t));
    int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    asm volatile("" : "+s"(w));
    tid = t;
    lane = t & 63;
    wave = w;
    g4 = lane >> 4;
    l16 = lane & 15;
    h2 = lane >> 5;
    l32 = lane & 31;
    wr0 = (w / W::NWC) * 64;
    wc0 = (w % W::NWC) * W::WC;
    sr = (TQ == 128) ? w : (w & 3);
    skb0 = (TQ == 128) ? 0 : 2 * (w >> 2);
    srow = sr * 16 + l16;
  };
  set_roles();

  // ---- persistent schedule.  Tiles are numbered with the column tile
  // fastest, then the row tile, the chunk and the head, so the tiles of one
  // chunk (which read the same state, keys and values) are consecutive.
  // Workgroup b runs on XCD b % 8; each XCD owns a contiguous eighth of the
  // tiles, and its G workgroups take G consecutive tiles per round (sharing
  // that XCD's L2), rotated by one each round so no workgroup always gets the
  // longest (last) row tile of a chunk.  With pair_tiles a workgroup instead
  // takes row tiles p and NQT-1-p of one chunk in two consecutive rounds:
  // every such pair covers the same number of key tiles, so the workgroups
  // of an XCD stay on the same few chunks and share their keys and values
  // in L2 instead of drifting apart.
  const int ntile = p.BH * NCB * NQT * NVT;
  const int G = gridDim.x;
  const bool xcd_split = (G & 7) == 0;
  const int gx = xcd_split ? G >> 3 : G;                  // workgroups per XCD
  const int x = xcd_split ? (int)blockIdx.x & 7 : 0;
  const int jw = xcd_split ? (int)blockIdx.x >> 3 : (int)blockIdx.x;
  const int per_x = xcd_split ? (ntile + 7) >> 3 : ntile;
  const int tbeg = x * per_x, tend = min(ntile, tbeg + per_x);
  // tile of round k for this workgroup, or -1 past the end; rows of a
  // ragged last chunk that hold no data are skipped
  const bool paired = p.pair_tiles && (NQT % 2) == 0;
  const int NPAIR = NQT / 2;
  const int nitem = ntile / 2;
  const int per_xi = xcd_split ? (nitem + 7) >> 3 : nitem;
  const int ibeg = x * per_xi, iend = min(nitem, ibeg + per_xi);
  auto tile_at = [&](int k) -> int {
    if (paired) {
      // work item = row tiles p and NQT-1-p of one (head, chunk, column
      // tile), in consecutive rounds: every item has the same key range
      const int it = ibeg + (k >> 1) * gx + jw;
      if (it >= iend) return -1;
      const int vt_ = it % NVT, pp = (it / NVT) % NPAIR, rest = it / (NVT * NPAIR);
      const int qt_ = (k & 1) ? NQT - 1 - pp : pp;
      return (rest * NQT + qt_) * NVT + vt_;
    }
    const int t = tbeg + k * gx + (jw + k) % gx;
    return t < tend ? t : (tbeg + k * gx < tend ? -2 : -1);
  };
  auto tile_live = [&](int t) -> bool {
    const int qt_ = (t / NVT) % NQT;
    const int c_ = c_lo + (t / (NVT * NQT)) % NCB;
    return qt_ * TQ < min(L, S - c_ * L);
  };
  int k_round = 0;
  auto next_tile = [&]() -> int {
    for (;;) {
      const int t = tile_at(k_round++);
      if (t == -1) return -1;
      if (t >= 0 && tile_live(t)) return t;
    }
  };

  // ---- requests for one tile, in the order they are needed (the memory
  // counter is waited on in issue order): gate terms and the normaliser, then
  // the Q tile.  The first chunk-state fragments follow at the top of the
  // tile.
  constexpr int GPT = (kMaxL + W::NT - 1) / W::NT;  // key positions per thread
  constexpr int NPT = (DK + W::NT - 1) / W::NT;
  constexpr int QPT = TQ * DK / 8 / W::NT;  // 16-byte Q loads per thread
  static_assert(TQ * DK / 8 % W::NT == 0, "Q tile split");
  constexpr int PD = W::CB >= 4 ? 1 : 3;  // k steps of state fragments loaded ahead
  float gu_r[GPT], n_r[NPT];
  float gb_r = 0.0f, gpm_r = 0.0f, mprev = 0.0f;
  uint4 qpre[QPT];
  uint4 bb[NKK][W::CB][2];
  // elements (bf16 words or int16 codes) per state
  constexpr size_t kStateElems = (size_t)DK * DV * (CODES ? 1 : 2);
  auto state_ptr = [&](int bh_, int c_) {
    return reinterpret_cast<const uint16_t*>(p.C_states) + ((size_t)bh_ * SL + c_ - c_lo) * kStateElems;
  };
  // Chunk-state fragments through a buffer resource: lane offset and the
  // wave's first 32-column block in one VGPR, the k step in a scalar offset
  // (a state is read whole, so every offset is in range), the column block
  // and plane as immediates.
  auto load_k = [&](__amdgpu_buffer_rsrc_t rs, int v0_, int kk) {
    if constexpr (CODES) {
      // fragment kk * (DV / 32) + nb at byte 1024 times that index
      const int voff = lane * 16 + ((v0_ + wc0) >> 5) * 1024;
#pragma unroll
      for (int cb = 0; cb < W::CB; ++cb) bb[kk][cb][0] = buf_load16_whole(rs, voff + cb * 1024, kk * DV * 32);
      return;
    }
    const int voff = lane * 16 + ((v0_ + wc0) >> 5) * 2048;
#pragma unroll
    for (int cb = 0; cb < W::CB; ++cb) {
      bb[kk][cb][0] = buf_load16_whole(rs, voff + cb * 2048, kk * DV * 64);
      if constexpr (SPLIT) bb[kk][cb][1] = buf_load16_whole(rs, voff + cb * 2048 + 1024, kk * DV * 64);
    }
  };
  auto state_rsrc = [&](int bh_, int c_) { return make_rsrc(state_ptr(bh_, c_), (uint32_t)(kStateElems * 2)); };
  auto request = [&](int t) {
    const int vt_ = t % NVT, qt_ = (t / NVT) % NQT;
    const int c_ = c_lo + (t / (NVT * NQT)) % NCB, bh_ = t / (NVT * NQT * NCB);
    const int t0_ = c_ * L, Lc_ = min(L, S - t0_), row0_ = qt_ * TQ, kend_ = min(row0_ + TQ, Lc_);
    const size_t gbase = (size_t)bh_ * S + t0_;
#pragma unroll
    for (int e = 0; e < GPT; ++e) gu_r[e] = tid + e * W::NT < kend_ ? p.gu2[gbase + tid + e * W::NT] : 0.0f;
    gb_r = gpm_r = 0.0f;
    if (tid < TQ && row0_ + tid < kend_) {
      gb_r = p.gb2[gbase + row0_ + tid];
      if constexpr (!SIG) gpm_r = p.gpm2[gbase + row0_ + tid];
    }
    if constexpr (!SIG) {
      mprev = p.m_states[(size_t)bh_ * SL + c_ - c_lo];
      const float* nst = p.n_states + ((size_t)bh_ * SL + c_ - c_lo) * DK;
#pragma unroll
      for (int e = 0; e < NPT; ++e) n_r[e] = tid + e * W::NT < DK ? nst[tid + e * W::NT] : 0.0f;
    }
    // the Q tile is contiguous; rows past the chunk read as zero (the step of
    // each load is in the lane offset, which the range check covers)
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(static_cast<const uint16_t*>(p.Q) + (gbase + row0_) * DK,
                                                (uint32_t)((Lc_ - row0_) * DK * 2));
#pragma unroll
    for (int i = 0; i < QPT; ++i) qpre[i] = buf_load16_nt(rq, tid * 16 + i * W::NT * 16);
  };

  int tile = next_tile();
  if (tile < 0) return;
  request(tile);

  for (;;) {
    __builtin_amdgcn_sched_barrier(0);
    set_roles();
    const int vt = tile % NVT;
    const int qt = (tile / NVT) % NQT;
    const int c = c_lo + (tile / (NVT * NQT)) % NCB;
    const int bh = tile / (NVT * NQT * NCB);
    const int v0 = vt * TV;
    const int t0 = c * L;
    const int Lc = min(L, S - t0);
    const int row0 = qt * TQ;
    const int kend = min(row0 + TQ, Lc);
    const bool srow_ok = row0 + srow < Lc;
    const uint16_t* K = static_cast<const uint16_t*>(p.K) + ((size_t)bh * S + t0) * DK;
    const uint16_t* V = static_cast<const uint16_t*>(p.V) + ((size_t)bh * S + t0) * DV + v0;
    const __amdgpu_buffer_rsrc_t rst = state_rsrc(bh, c);
#pragma unroll
    for (int kk = 0; kk < PD && kk < NKK; ++kk) load_k(rst, v0, kk);
    __builtin_amdgcn_sched_barrier(0);
    // scales of this wave's fragments (int16-coded states): wave-uniform
    float scl[CODES ? NKK : 1][CODES ? W::CB : 1];
    if constexpr (CODES) {
      const int f0 = __builtin_amdgcn_readfirstlane(
          (int)(((size_t)bh * SL + c - c_lo) * (DK / 16) * (DV / 32)) + ((v0 + wc0) >> 5));
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
        for (int cb = 0; cb < W::CB; ++cb) scl[kk][cb] = p.C_scales[f0 + kk * (DV / 32) + cb];
    }

    // ---- gate terms of this chunk (log2 units, written by the gates kernel):
    // u for the keys [0, kend); b and the running max of u for this tile's rows.
#pragma unroll
    for (int e = 0; e < GPT; ++e)
      if (tid + e * W::NT < kend) s_u2[tid + e * W::NT] = gu_r[e];
    if (tid < TQ) {
      if (row0 + tid < kend) {
        const float b2 = gb_r;
        if constexpr (SIG) {
          s_row_r2[tid] = b2;
          s_row_w[tid] = exp2f(b2);
          s_row_m2[tid] = 0.0f;
        } else {
          const float M2 = mprev * kLog2e;
          const float mx = fmaxf(M2, gpm_r);
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
#pragma unroll
      for (int e = 0; e < NPT; ++e)
        if (tid + e * W::NT < DK) s_n[tid + e * W::NT] = n_r[e];
    }
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int idx = tid + i * W::NT;
      const int rr = idx / (DK / 8), cc = (idx % (DK / 8)) * 8;
      *reinterpret_cast<uint4*>(s_q + rr * W::LDQ + cc) = qpre[i];
    }
    __syncthreads();

    float16_t acc[2][W::CB];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int cb = 0; cb < W::CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[rb][cb][r] = 0.0f;

    // ---- inter-chunk term: acc = Q . C with the packed state fragments; the Q
    // rows use the same contraction-slot order as the packed state.
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      if (kk + PD < NKK) load_k(rst, v0, kk + PD);
      // keep the prefetch ahead of this step's products (the scheduler would
      // otherwise sink the loads next to their use to save registers)
      __builtin_amdgcn_sched_barrier(0);
      bf16x8_t qa[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const uint16_t* qp = s_q + (wr0 + 32 * rb + l32) * W::LDQ + 16 * kk + 4 * h2;
        const uint2 x0 = *reinterpret_cast<const uint2*>(qp);
        const uint2 x1 = *reinterpret_cast<const uint2*>(qp + 8);
        qa[rb] = as_bf16x8(make_uint4(x0.x, x0.y, x1.x, x1.y));
      }
#pragma unroll
      for (int cb = 0; cb < W::CB; ++cb) {
        uint4 ph = bb[kk][cb][0], pl;
        if constexpr (!CODES && SPLIT) pl = bb[kk][cb][1];
        if constexpr (CODES) {
          const uint32_t cw[4] = {ph.x, ph.y, ph.z, ph.w};
          uint32_t hw[4], lw[4];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            split_bf16x2((float)((int)(cw[q] << 16) >> 16) * scl[kk][cb], (float)((int)cw[q] >> 16) * scl[kk][cb],
                         hw[q], lw[q]);
          ph = make_uint4(hw[0], hw[1], hw[2], hw[3]);
          pl = make_uint4(lw[0], lw[1], lw[2], lw[3]);
        }
        const bf16x8_t bh_ = as_bf16x8(ph);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) acc[rb][cb] = mma32b(qa[rb], bh_, acc[rb][cb]);
        if constexpr (SPLIT) {
          const bf16x8_t bl_ = as_bf16x8(pl);
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) acc[rb][cb] = mma32b(qa[rb], bl_, acc[rb][cb]);
        }
      }
    }
    // this lane's Q row as B fragments of the transposed score tile
    uint4 qs[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qs[ks] = *reinterpret_cast<const uint4*>(s_q + srow * W::LDQ + 32 * ks + 8 * g4);
    __syncthreads();  // the Q tile's LDS is reused for K, P and V below
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

    // normaliser contribution of the state: s e^{b + M - m} q . n
    float den_part = 0.0f;
    if constexpr (!SIG) {
      if (skb0 == 0 && srow_ok) {
        float d = 0.0f;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const uint4 u = qs[ks];
          const uint32_t ww[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            d += __uint_as_float(ww[e] << 16) * s_n[32 * ks + 8 * g4 + 2 * e];
            d += __uint_as_float(ww[e] & 0xffff0000u) * s_n[32 * ks + 8 * g4 + 2 * e + 1];
          }
        }
        den_part = d * scale * s_row_w[srow];
      }
    }

    // ---- intra-chunk term over key tiles [0, kend)
    const float r2 = s_row_r2[srow];
    const int tau = row0 + srow;
    const int ntiles = (kend + W::TKV - 1) / W::TKV;
    // K and V tiles (64 rows) are prefetched into registers one tile ahead.
    constexpr int KPT = W::TKV * DK / 8 / W::NT;  // 16-byte K loads per thread
    constexpr int VPT = W::TKV * TV / 8 / W::NT;  // 16-byte V loads per thread
    static_assert(W::TKV * DK / 8 % W::NT == 0 && W::TKV * TV / 8 % W::NT == 0, "tile split");
    uint4 kpre[KPT], vpre[VPT];
    // K and V of this chunk through buffer resources: rows past the chunk
    // read as zero.  The tile start moves each resource's base; the step of
    // the thread's i-th load is in its lane offset.
    const uint32_t kext = (uint32_t)(Lc * DK * 2);
    const uint32_t vext = (uint32_t)((Lc - 1) * DV * 2 + TV * 2);
    const int vvoff = (tid / (TV / 8)) * DV * 2 + (tid % (TV / 8)) * 16;
    auto load_kv = [&](int s0) {
      const __amdgpu_buffer_rsrc_t rk = make_rsrc_at(K, kext, s0 * DK * 2);
      const __amdgpu_buffer_rsrc_t rv = make_rsrc_at(V, vext, s0 * DV * 2);
#pragma unroll
      for (int i = 0; i < KPT; ++i) kpre[i] = buf_load16(rk, tid * 16 + i * W::NT * 16);
#pragma unroll
      for (int i = 0; i < VPT; ++i) vpre[i] = buf_load16(rv, vvoff + i * (W::NT / (TV / 8)) * DV * 2);
    };
    if (ntiles > 0) load_kv(0);

    for (int j = 0; j < ntiles; ++j) {
      const int s0 = j * W::TKV;
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int idx = tid + i * W::NT;
        const int rr = idx / (DK / 8), cc = (idx % (DK / 8)) * 8;
        *reinterpret_cast<uint4*>(s_k + rr * W::LDK + cc) = kpre[i];
      }
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int idx = tid + i * W::NT;
        const int rr = idx / (TV / 8), cc = (idx % (TV / 8)) * 8;
        *reinterpret_cast<uint4*>(s_v + rr * W::LDV + cc) = vpre[i];
      }
      if (j + 1 < ntiles) load_kv(s0 + W::TKV);
      __syncthreads();

      // transposed scores for 16 rows x SKB key blocks; P to LDS as hi/lo planes
      float4_t sacc[W::SKB];
      bool live[W::SKB];
      bool all_live = true;
#pragma unroll
      for (int kb = 0; kb < W::SKB; ++kb) {
        const int key0 = s0 + 16 * (skb0 + kb);
        sacc[kb] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
        live[kb] = key0 <= row0 + sr * 16 + 15 && key0 < kend;  // wave-uniform
        all_live = all_live && live[kb];
      }
      if (all_live) {
        // independent accumulation chains, interleaved
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
          for (int kb = 0; kb < W::SKB; ++kb) {
            const uint4 a = *reinterpret_cast<const uint4*>(s_k + (16 * (skb0 + kb) + l16) * W::LDK + 32 * ks + 8 * g4);
            sacc[kb] = mma16b(as_bf16x8(a), as_bf16x8(qs[ks]), sacc[kb]);
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < W::SKB; ++kb) {
          if (!live[kb]) continue;
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            const uint4 a = *reinterpret_cast<const uint4*>(s_k + (16 * (skb0 + kb) + l16) * W::LDK + 32 * ks + 8 * g4);
            sacc[kb] = mma16b(as_bf16x8(a), as_bf16x8(qs[ks]), sacc[kb]);
          }
        }
      }
#pragma unroll
      for (int kb = 0; kb < W::SKB; ++kb) {
        const int sb = skb0 + kb;
        const int key0 = s0 + 16 * sb;
        const float4 u4 = *reinterpret_cast<const float4*>(s_u2 + key0 + 4 * g4);
        const float uu[4] = {u4.x, u4.y, u4.z, u4.w};
        float val[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int sg = key0 + 4 * g4 + r;
          const float pv = scale * sacc[kb][r] * __builtin_amdgcn_exp2f(r2 + uu[r]);
          val[r] = (live[kb] && sg <= tau && tau < kend) ? pv : 0.0f;
          den_part += val[r];
        }
        uint2 ph, pl;
        if constexpr (SPLIT) {
          split_bf16x2(val[0], val[1], ph.x, pl.x);
          split_bf16x2(val[2], val[3], ph.y, pl.y);
          *reinterpret_cast<uint2*>(s_pl + srow * W::LDP + 16 * sb + 4 * g4) = pl;
        } else {
          ph.x = round_bf16x2(val[0], val[1]);
          ph.y = round_bf16x2(val[2], val[3]);
        }
        *reinterpret_cast<uint2*>(s_ph + srow * W::LDP + 16 * sb + 4 * g4) = ph;
      }
      __syncthreads();

      // acc += P . V over 16-key steps
#pragma unroll
      for (int kk = 0; kk < W::TKV / 16; ++kk) {
        const int key0 = s0 + 16 * kk;
        if (key0 > row0 + wr0 + 63 || key0 >= kend) continue;  // wave-uniform: all zero
        uint4 ah[2], al[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          ah[rb] = frag_row_u(s_ph, W::LDP, wr0 + 32 * rb, 16 * kk, lane);
          if constexpr (SPLIT) al[rb] = frag_row_u(s_pl, W::LDP, wr0 + 32 * rb, 16 * kk, lane);
        }
#pragma unroll
        for (int cb = 0; cb < W::CB; ++cb) {
          const bf16x8_t bv = as_bf16x8(frag_tr_u(s_v, W::LDV, 16 * kk, wc0 + 32 * cb, lane));
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            acc[rb][cb] = mma32b(as_bf16x8(ah[rb]), bv, acc[rb][cb]);
            if constexpr (SPLIT) acc[rb][cb] = mma32b(as_bf16x8(al[rb]), bv, acc[rb][cb]);
          }
        }
      }
      __syncthreads();
    }

    // the next tile's gate terms and Q tile are requested now and land
    // while this tile's epilogue runs
    const int next = next_tile();
    if (next >= 0) request(next);
    __builtin_amdgcn_sched_barrier(0);

    // ---- normaliser per row, then H
    if constexpr (!SIG) {
      den_part += __shfl_xor(den_part, 16, 64);
      den_part += __shfl_xor(den_part, 32, 64);
      if (g4 == 0) {
        if (TQ == 128 || skb0 == 0) s_row_den[srow] = den_part;
        else s_den2[srow] = den_part;
      }
      __syncthreads();
      if (tid < TQ) {
        float d = s_row_den[tid];
        if (TQ != 128) d += s_den2[tid];
        s_row_den[tid] = d;
        // reciprocal of the normaliser, reused for every column of the row
        s_den2[tid] = 1.0f / (fmaxf(fabsf(d), exp2f(-s_row_m2[tid])) + p.eps);
      }
    }
    __syncthreads();
    // H through a buffer resource spanning this chunk's rows: stores to rows
    // past the chunk fall outside it and are dropped.  Each accumulator
    // register holds one row of 32 consecutive columns across a half-wave, so
    // each store writes two full 128-byte row segments; the row offsets are
    // compile-time multiples of DV added to the lane offset.
    auto store_h = [&](auto esize) {
      constexpr int E = decltype(esize)::value;
      const __amdgpu_buffer_rsrc_t rh = make_rsrc(static_cast<const char*>(p.H) + ((size_t)bh * S + t0) * DV * E,
                                                  (uint32_t)(Lc * DV * E));
      // float32: one value per lane and store.  bf16: lane pairs (l32 even,
      // odd) swap values so that each lane holds two adjacent columns of one
      // row (the even lane rows q = 0, 2, the odd lane rows 1, 3), rounded
      // together and stored as one word (measured 3 % faster than one 2-byte
      // store per value; the same exchange with 8-byte float32 stores was 6 %
      // slower)
      const bool odd = (l32 & 1) != 0;
      const int hvoff = E == 2 ? ((row0 + wr0 + 4 * h2 + (odd ? 1 : 0)) * DV + v0 + wc0 + (l32 & ~1)) * E
                               : ((row0 + wr0 + 4 * h2) * DV + v0 + wc0 + l32) * E;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int rowl = 32 * rb + 8 * r4;  // + 4 * h2 + q: row within the wave's 64
          float4 inv = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
          if constexpr (!SIG) inv = *reinterpret_cast<const float4*>(s_den2 + wr0 + rowl + 4 * h2);
          const float invq[4] = {inv.x, inv.y, inv.z, inv.w};
          // non-temporal (aux 2): H is not read again here, so it should not
          // push the state and K/V lines of sibling row tiles out of L2
          if constexpr (E == 2) {
#pragma unroll
            for (int cb = 0; cb < W::CB; ++cb) {
              float hv[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) hv[q] = acc[rb][cb][4 * r4 + q] * invq[q];
#pragma unroll
              for (int qp = 0; qp < 2; ++qp) {
                const float2 pr = pair_rows_to_cols(hv[2 * qp], hv[2 * qp + 1], odd);
                __builtin_amdgcn_raw_buffer_store_b32(round_bf16x2(pr.x, pr.y), rh,
                                                      hvoff + ((rowl + 2 * qp) * DV + 32 * cb) * E, 0, 2);
              }
            }
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int hro = hvoff + (rowl + q) * DV * E;
#pragma unroll
              for (int cb = 0; cb < W::CB; ++cb)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[rb][cb][4 * r4 + q] * invq[q]), rh,
                                                      hro + 32 * cb * E, 0, 2);
            }
          }
        }
    };
    // Backward recompute (exp gate, whole rows per workgroup): instead of H,
    // the row terms of the gradient, from dh . h with h = acc / z.
    auto store_delta = [&](auto dsize) {
      constexpr int E = decltype(dsize)::value;  // bytes per dH element
      const __amdgpu_buffer_rsrc_t rd = make_rsrc(static_cast<const char*>(p.dH) + ((size_t)bh * S + t0) * DV * E,
                                                  (uint32_t)(Lc * DV * E));
      const int dvoff = ((row0 + wr0 + 4 * h2) * DV + v0 + wc0 + l32) * E;
      // this lane's partial sums over its columns, slot j = 16 rb + 4 r4 + q
      // for row wr0 + 32 rb + 8 r4 + 4 h2 + q
      float part[32];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int rowl = 32 * rb + 8 * r4;
          const float4 inv = *reinterpret_cast<const float4*>(s_den2 + wr0 + rowl + 4 * h2);
          const float invq[4] = {inv.x, inv.y, inv.z, inv.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int dro = dvoff + (rowl + q) * DV * E;
            float d = 0.0f;
#pragma unroll
            for (int cb = 0; cb < W::CB; ++cb) {
              float dh;
              if constexpr (E == 2)
                dh = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rd, dro + 32 * cb * E, 0, 0) << 16);
              else
                dh = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rd, dro + 32 * cb * E, 0, 0));
              d += dh * acc[rb][cb][4 * r4 + q];
            }
            part[16 * rb + 4 * r4 + q] = d * invq[q];
          }
        }
      // butterfly over the 32 lanes of each half-wave: after the step with
      // offset o, a lane keeps the half of its slots whose bit o matches its
      // lane bit; at the end lane l32 holds the sum of slot l32
#pragma unroll
      for (int n = 32, o = 16; o >= 1; n >>= 1, o >>= 1) {
        const bool up = (l32 & o) != 0;
#pragma unroll
        for (int j = 0; j < n / 2; ++j) {
          const float send = up ? part[j] : part[j + n / 2];
          const float keep = up ? part[j + n / 2] : part[j];
          part[j] = keep + __shfl_xor(send, o, 64);
        }
      }
      // slot l32 = 16 rb + 4 r4 + q: row wr0 + 32 rb + 8 r4 + 4 h2 + q
      const int rl = wr0 + 32 * (l32 >> 4) + 8 * ((l32 >> 2) & 3) + 4 * h2 + (l32 & 3);
      float* const s_dp = reinterpret_cast<float*>(s_buf);  // [column wave][row], the K/P/V space is free
      s_dp[(wave % W::NWC) * TQ + rl] = part[0];
      __syncthreads();
      if (tid < TQ && row0 + tid < Lc) {
        float d = 0.0f;
#pragma unroll
        for (int w = 0; w < W::NWC; ++w) d += s_dp[w * TQ + tid];
        const float den = s_row_den[tid], invz = s_den2[tid];
        const size_t ro = (size_t)bh * S + t0 + row0 + tid;
        p.ginvz[ro] = invz;
        p.gdelta[ro] = fabsf(den) > exp2f(-s_row_m2[tid]) ? (den > 0.0f ? -d * invz : d * invz) : 0.0f;
      }
    };
    if constexpr (DELTA) {
      if (p.dh_bf16) store_delta(std::integral_constant<int, 2>{});
      else store_delta(std::integral_constant<int, 4>{});
    } else if (p.h_bf16) {
      store_h(std::integral_constant<int, 2>{});
    } else {
      store_h(std::integral_constant<int, 4>{});
    }
    if constexpr (!SIG) {
      if (vt == 0 && tid < TQ && row0 + tid < Lc) {
        const size_t ro = (size_t)bh * S + t0 + row0 + tid;
        if (p.m_rows) p.m_rows[ro] = s_row_m2[tid] * kLn2;
        if (p.den_rows) p.den_rows[ro] = s_row_den[tid];
      }
    }
    if (next < 0) break;
    tile = next;
    __syncthreads();  // the epilogue's LDS reads precede the next tile's writes
  }
}

template <int DK, int DV, int TQ, int TV, bool SIG, bool SPLIT>
hipError_t launch_t(const HintraParams& p0, hipStream_t stream) {
  // Long chunks (8 or more row tiles) pair their row tiles: measured on the
  // long-context workload (chunk 1024, 128-row tiles) the L2 re-fetch of K
  // and V halves (6.45 -> 3.85 GB per launch) and the kernel gains 4 %; with
  // 4 row tiles per chunk the unpaired rotation is faster.
  HintraParams p = p0;
  p.pair_tiles = p.L / TQ >= 8;
  // One workgroup per CU walks the tiles (the LDS footprint allows one per
  // CU); fewer when there are fewer tiles.
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const long long ntile = (long long)p.BH * ((p.c_hi < 0 ? p.Nc : p.c_hi) - p.c_lo) * (p.L / TQ) * (DV / TV);
  dim3 grid((unsigned)(ntile < cus ? ntile : cus));
  if constexpr (!SIG && TV == DV) {
    if (p.dH) {
      hipLaunchKernelGGL((hintra_wide_kernel<DK, DV, TQ, TV, SIG, SPLIT, true>), grid, dim3(512), 0, stream, p);
      return hipGetLastError();
    }
  }
  if (p.dH) return hipErrorInvalidValue;  // the row terms need whole rows and the exp gate
  if (p.C_scales) {
    if constexpr (SPLIT) {
      hipLaunchKernelGGL((hintra_wide_kernel<DK, DV, TQ, TV, SIG, SPLIT, false, true>), grid, dim3(512), 0, stream,
                         p);
      return hipGetLastError();
    }
    return hipErrorInvalidValue;  // int16-coded states feed the split forward only
  }
  hipLaunchKernelGGL((hintra_wide_kernel<DK, DV, TQ, TV, SIG, SPLIT>), grid, dim3(512), 0, stream, p);
  return hipGetLastError();
}

// Tile choice: 64-row tiles span all DV columns; 128-row tiles span DV / 2
// columns when DV = 512 (keeps 64 accumulators per lane).
template <int DK, int DV, bool SIG, bool SPLIT>
hipError_t launch_tq(const HintraParams& p, hipStream_t stream) {
  if (p.tile_lq == 128) {
    if constexpr (DV == 512) return launch_t<DK, DV, 128, 256, SIG, SPLIT>(p, stream);
    else return launch_t<DK, DV, 128, DV, SIG, SPLIT>(p, stream);
  }
  if constexpr (DV >= 256) return launch_t<DK, DV, 64, DV, SIG, SPLIT>(p, stream);
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
