// Inter-chunk recurrence, wide-tile version for bf16 inputs (gfx950).
//
// Same recurrence as states_kernel.hip (TFLA abstract: chunkwise-parallel
// form with states carried between chunks), in log2 units on the gate terms
// that gates_kernel.hip leaves per position (b: in-chunk cumulative
// log-forget sum, u = i~ - b, pm: running max of u):
//   M' = g + max(M, pm_last),  g = b_last
//   C' = 2^{g + M - M'} C + sum_t 2^{g + u_t - M'} k_t v_t^T,   n' likewise
//   (sigmoid gate: no M; C' = 2^{g} C + sum_t 2^{g + u_t} k_t v_t^T)
// Organisation:
//   * one workgroup (4 waves) keeps a TK x TV tile of C in 32x32x16 bf16
//     matrix-core accumulators (float32) for the whole sequence (TK = TV = 64
//     or 128);
//   * each 64-step time block stages the gated keys as bf16 hi + lo planes
//     (computed in float32) and the values unchanged, both row-major in LDS,
//     and reads them transposed with ds_read_b64_tr_b16 (the contraction runs
//     over time, down the rows);
//   * the state entering every chunk is written in the packed layout the
//     intra-chunk kernel consumes (see pack_offset): for every 16-row k step
//     and 32-column block, 64 lanes x 8 bf16 values, hi plane then lo plane.
//     The lane and slot order is the accumulator's own, so the writes are
//     plain 16-byte stores.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace mlstm {
namespace {

constexpr int kMaxL = 1024;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kTT = 64;  // time steps per LDS stage

template <int TK, int TV, bool SIG, bool SPLIT>
__global__ __launch_bounds__(256) void states_wide_kernel(const StatesParams p) {
  constexpr int WR = TK / 2, WCOL = TV / 2;      // wave tile
  constexpr int RB = WR / 32, CB = WCOL / 32;    // 32x32 blocks per wave
  // row strides of 16 banks mod 64 keep apart the 4 rows x 64 bytes that a
  // half-wave takes in one transposing read
  constexpr int LDK = TK + 32, LDV = TV + 32;
  constexpr int KSEG = TK / 8, VSEG = TV / 8;    // 16-byte segments per row
  constexpr int KPT = kTT * KSEG / 256, VPT = kTT * VSEG / 256;
  static_assert(kTT * KSEG % 256 == 0 && kTT * VSEG % 256 == 0, "staging split");

  __shared__ float s_w[kMaxL];
  __shared__ float s_np[256 / KSEG][TK];
  __shared__ __align__(16) uint16_t s_kh[kTT * LDK];
  __shared__ __align__(16) uint16_t s_kl[kTT * LDK];
  __shared__ __align__(16) uint16_t s_v[kTT * LDV];

  const int NTK = p.DK / TK, NTV = p.DV / TV;
  const int bid = blockIdx.x;
  const int bh = bid % p.BH;
  const int kt = (bid / p.BH) % NTK;
  const int vt = bid / (p.BH * NTK);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h2 = lane >> 5, l32 = lane & 31;
  const int S = p.S, DK = p.DK, DV = p.DV, L = p.L, Nc = p.Nc;
  const int wr0 = (wave >> 1) * WR, wc0 = (wave & 1) * WCOL;  // inside the tile
  const uint16_t* K = static_cast<const uint16_t*>(p.K) + (size_t)bh * S * DK + kt * TK;
  const uint16_t* V = static_cast<const uint16_t*>(p.V) + (size_t)bh * S * DV + vt * TV;
  const bool own_n = !SIG && vt == 0;
  const int nseg = tid % KSEG;     // this thread's key segment while staging
  const int nrow = tid / KSEG;     // and its first time row

  float16_t acc[RB][CB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int krow = kt * TK + wr0 + 32 * rb + 8 * (r >> 2) + 4 * h2 + (r & 3);
        const int vcol = vt * TV + wc0 + 32 * cb + l32;
        acc[rb][cb][r] = p.C0 ? p.C0[(size_t)bh * DK * DV + (size_t)krow * DV + vcol] : 0.0f;
      }
  float nreg = 0.0f;  // n for key row kt*TK + tid (tid < TK), own_n only
  if (own_n && tid < TK && p.n0) nreg = p.n0[(size_t)bh * DK + kt * TK + tid];
  float M2 = 0.0f;  // stabiliser in log2 units
  if (!SIG && p.m0) M2 = p.m0[bh] * kLog2e;
  // gate terms of the next chunk: u for positions 4 tid .. 4 tid + 3, then
  // b and the running max of u at the chunk's last position
  float gnext[6];
  auto load_gates = [&](int cc) {
    const int tc = cc * L;
    const int Lcc = min(L, S - tc);
    const float* gu = p.gu2 + (size_t)bh * S + tc;
#pragma unroll
    for (int e = 0; e < 4; ++e) gnext[e] = 4 * tid + e < Lcc ? gu[4 * tid + e] : 0.0f;
    gnext[4] = p.gb2[(size_t)bh * S + tc + Lcc - 1];
    gnext[5] = SIG ? 0.0f : p.gpm2[(size_t)bh * S + tc + Lcc - 1];
  };
  if (Nc > 0) load_gates(0);

  uint4 kpre[KPT], vpre[VPT];
  auto load_kv = [&](int t0, int tb, int Lc) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int t = nrow + i * (256 / KSEG);
      kpre[i] = (tb + t < Lc) ? *reinterpret_cast<const uint4*>(K + (size_t)(t0 + tb + t) * DK + nseg * 8)
                              : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int idx = tid + i * 256;
      const int t = idx / VSEG, sg = idx % VSEG;
      vpre[i] = (tb + t < Lc) ? *reinterpret_cast<const uint4*>(V + (size_t)(t0 + tb + t) * DV + sg * 8)
                              : make_uint4(0, 0, 0, 0);
    }
  };

  for (int c = 0; c <= Nc; ++c) {
    // ---- state entering chunk c, packed hi/lo fragments
    {
      uint16_t* P = reinterpret_cast<uint16_t*>(p.C_states) + ((size_t)bh * (Nc + 1) + c) * DK * DV * 2;
      const int NB = DV / 32;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const int kblk = (kt * TK + wr0 + 32 * rb) / 32;
          const int nblk = (vt * TV + wc0 + 32 * cb) / 32;
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              split_bf16x2(acc[rb][cb][8 * half + 2 * e], acc[rb][cb][8 * half + 2 * e + 1], hi[e], lo[e]);
            const size_t blk = ((size_t)(2 * kblk + half) * NB + nblk) * 2;
            *reinterpret_cast<uint4*>(P + (blk + 0) * 512 + lane * 8) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
            *reinterpret_cast<uint4*>(P + (blk + 1) * 512 + lane * 8) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
          }
        }
      if (own_n && tid < TK) p.n_states[((size_t)bh * (Nc + 1) + c) * DK + kt * TK + tid] = nreg;
      if (!SIG && kt == 0 && vt == 0 && tid == 0) p.m_states[(size_t)bh * (Nc + 1) + c] = M2 * kLn2;
    }
    if (c == Nc) break;

    const int t0 = c * L;
    const int Lc = min(L, S - t0);
    load_kv(t0, 0, Lc);  // first time block
    // ---- gate weights from the per-position gate terms (log2 units), which
    // were requested one chunk ahead: M' = g + max(M, pm_last),
    // w_tau = 2^{g + u_tau - M'}, decay of the carried state 2^{g + M - M'}.
    const float g2 = gnext[4], umax2 = gnext[5];
    float uc[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) uc[e] = gnext[e];
    if (c + 1 < Nc) load_gates(c + 1);
    float decay, Mn2 = 0.0f;
    if constexpr (SIG) {
      decay = exp2f(g2);
    } else {
      Mn2 = g2 + fmaxf(M2, umax2);
      decay = exp2f(g2 + M2 - Mn2);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int pos = 4 * tid + e;
      s_w[pos] = pos < Lc ? exp2f(g2 + uc[e] - Mn2) : 0.0f;
    }
    M2 = Mn2;
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) acc[rb][cb] *= decay;
    float np[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) np[e] = 0.0f;

    for (int tb = 0; tb < Lc; tb += kTT) {
      // stage gated keys (hi/lo) and values
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int t = nrow + i * (256 / KSEG);
        const float w = s_w[tb + t];  // 0 beyond the chunk
        const uint32_t ww[4] = {kpre[i].x, kpre[i].y, kpre[i].z, kpre[i].w};
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = __uint_as_float(ww[e] << 16) * w;
          const float x1 = __uint_as_float(ww[e] & 0xffff0000u) * w;
          np[2 * e] += x0;
          np[2 * e + 1] += x1;
          if constexpr (SPLIT) split_bf16x2(x0, x1, hi[e], lo[e]);
          else hi[e] = round_bf16x2(x0, x1);
        }
        *reinterpret_cast<uint4*>(s_kh + t * LDK + nseg * 8) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        if constexpr (SPLIT) *reinterpret_cast<uint4*>(s_kl + t * LDK + nseg * 8) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
      }
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int idx = tid + i * 256;
        const int t = idx / VSEG, sg = idx % VSEG;
        *reinterpret_cast<uint4*>(s_v + t * LDV + sg * 8) = vpre[i];
      }
      if (tb + kTT < Lc) load_kv(t0, tb + kTT, Lc);
      __syncthreads();
#pragma unroll
      for (int ks = 0; ks < kTT / 16; ++ks) {
        if (tb + 16 * ks >= Lc) break;  // uniform: rest of the block is padding
        bf16x8_t ah[RB], al[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          ah[rb] = as_bf16x8(frag_tr_u(s_kh, LDK, 16 * ks, wr0 + 32 * rb, lane));
          if constexpr (SPLIT) al[rb] = as_bf16x8(frag_tr_u(s_kl, LDK, 16 * ks, wr0 + 32 * rb, lane));
        }
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const bf16x8_t bv = as_bf16x8(frag_tr_u(s_v, LDV, 16 * ks, wc0 + 32 * cb, lane));
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            acc[rb][cb] = mma32b(ah[rb], bv, acc[rb][cb]);
            if constexpr (SPLIT) acc[rb][cb] = mma32b(al[rb], bv, acc[rb][cb]);
          }
        }
      }
      __syncthreads();
    }
    if (own_n) {
      // n' = decay n + sum_t w_t k_t: reduce the per-thread partial sums
#pragma unroll
      for (int e = 0; e < 8; ++e) s_np[nrow][nseg * 8 + e] = np[e];
      __syncthreads();
      if (tid < TK) {
        float sacc = 0.0f;
        for (int r = 0; r < 256 / KSEG; ++r) sacc += s_np[r][tid];
        nreg = nreg * decay + sacc;
      }
      __syncthreads();
    }
  }

  if (p.C_out) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int krow = kt * TK + wr0 + 32 * rb + 8 * (r >> 2) + 4 * h2 + (r & 3);
          const int vcol = vt * TV + wc0 + 32 * cb + l32;
          p.C_out[(size_t)bh * DK * DV + (size_t)krow * DV + vcol] = acc[rb][cb][r];
        }
  }
  if (own_n && p.n_out && tid < TK) p.n_out[(size_t)bh * DK + kt * TK + tid] = nreg;
  if (!SIG && p.m_out && kt == 0 && vt == 0 && tid == 0) p.m_out[bh] = M2 * kLn2;
}

// Row-tile variant for many heads: a workgroup of 8 waves keeps a TK x DV
// tile of C (each wave a 64 x 64 block) for the whole sequence, so each gated
// key block is staged once for all value columns.  The tiles of one head are
// placed on one XCD (they read the same V rows at about the same time).
// Software pipeline over 32-step blocks of the flattened (chunk, step)
// sequence:
//   * LDS holds two stages: block j is in the matrix cores while block j+1 is
//     written, one barrier per block;
//   * the global loads of block j+2 are in flight meanwhile (two register
//     sets, issued two blocks ahead);
//   * each staging thread forms the gate weight of its own time row from the
//     per-position gate terms; the chunk stabiliser and decay are formed when
//     a chunk's first block is staged and applied one block later, when the
//     matrix cores reach it.
// PLAIN: the states go out as float32 row-major (StatesParams::C_plain)
// instead of packed, for a reader other than the intra-chunk kernel.
// CODES: the packed states go out as int16 codes with one power-of-two scale
// per 16 x 32 fragment (StatesParams::C_scales), half the bytes of the hi +
// lo pair.
template <int TK, int TV, bool SIG, bool SPLIT, bool PLAIN = false, bool CODES = false>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void states_rows_kernel(
    const StatesParams p) {
  constexpr int NT = 512, NW = 8, TB = 32;
  constexpr int NWC = TV / 64;
  static_assert((TK / 64) * NWC == NW, "eight 64x64 wave tiles");
  constexpr int LDK = TK + 32, LDV = TV + 32;  // 16 banks mod 64 (see above)
  constexpr int EPT = TB * TK / NT;  // key elements per thread and block
  constexpr int TPR = TK / EPT;      // staging threads per time row
  static_assert(TPR == 16 && (EPT == 4 || EPT == 8), "staging split");
  constexpr int VSEG = TV / 8;
  constexpr int VPT = TB * VSEG / NT;  // 16-byte V loads per thread and block
  static_assert(TB * VSEG % NT == 0, "V staging split");
  constexpr int KBUF = TB * LDK, VBUF = TB * LDV;
  typedef typename std::conditional<EPT == 4, uint2, uint4>::type KVec;

  __shared__ float s_np[NW][TK];
  __shared__ __align__(16) uint16_t s_kh[2 * KBUF];
  __shared__ __align__(16) uint16_t s_kl[SPLIT ? 2 * KBUF : 8];
  __shared__ __align__(16) uint16_t s_v[2 * VBUF];

  const int NTK = p.DK / TK;
  const int nblk = gridDim.x;
  int bid = blockIdx.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int kt = bid % NTK;
  const int seg = (bid / NTK) % p.nseg;
  const int bh = bid / (NTK * p.nseg);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h2 = lane >> 5, l32 = lane & 31;
  const int S = p.S, DK = p.DK, L = p.L, Nc = p.Nc;
  constexpr int DV = TV;
  // Chunks [c_beg, c_end) of this head.  With several segments, segment 0 starts
  // from the initial state and later ones from zero (stabiliser -inf); their
  // chunk states are local and the join kernels turn them into the true ones.
  const bool segmented = p.nseg > 1;
  // Chunks [c_lo, c_hi) of this launch (all of them unless the forward runs
  // in blocks of chunks); the state entering chunk c sits at slot c - c_lo of
  // the head's SL slots.
  const int c_hi = p.c_hi < 0 ? Nc : p.c_hi;
  const int SL = p.slots ? p.slots : Nc + 1;
  const int c_beg = p.c_lo + seg * p.cps;
  const int c_end = min(c_hi, c_beg + p.cps);
  const int wr0 = (wave / NWC) * 64, wc0 = (wave % NWC) * 64;  // inside the tile
  const uint16_t* K = static_cast<const uint16_t*>(p.K) + (size_t)bh * S * DK + kt * TK;
  const uint16_t* V = static_cast<const uint16_t*>(p.V) + (size_t)bh * S * DV;
  const size_t gbase = (size_t)bh * S;
  const int krs = tid / TPR, kcs = (tid % TPR) * EPT;  // staging row and columns

  float16_t acc[2][2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int krow = kt * TK + wr0 + 32 * rb + 8 * (r >> 2) + 4 * h2 + (r & 3);
        const int vcol = wc0 + 32 * cb + l32;
        acc[rb][cb][r] = (p.C0 && seg == 0) ? p.C0[(size_t)bh * DK * DV + (size_t)krow * DV + vcol] : 0.0f;
      }
  float nreg = 0.0f;  // n for key row kt * TK + tid (tid < TK)
  if (!SIG && tid < TK && p.n0 && seg == 0) nreg = p.n0[(size_t)bh * DK + kt * TK + tid];
  float Mst2 = 0.0f;  // stabiliser (log2 units) after the last chunk begun by the staging side
  if (!SIG && p.m0) Mst2 = p.m0[bh] * kLog2e;
  if (!SIG && seg > 0) Mst2 = -INFINITY;

  auto write_state = [&](int entry, float M2) __attribute__((always_inline)) {
    if constexpr (PLAIN) {
      // float32 row-major copy: a half-wave stores 128 contiguous bytes of a row
      float* Pl = p.C_plain + ((size_t)bh * SL + entry - p.c_lo) * DK * DV;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int krow = kt * TK + wr0 + 32 * rb + 8 * (r >> 2) + 4 * h2 + (r & 3);
            __builtin_nontemporal_store(acc[rb][cb][r], Pl + (size_t)krow * DV + wc0 + 32 * cb + l32);
          }
    }
    constexpr int NB = DV / 32;
    if constexpr (CODES) {
      // Fragment f = 2 kblk + half, nb holds exactly this wave's eight values
      // per lane of one (rb, cb, half): its scale is a power of two between
      // its largest magnitude over 32767 and twice that, so that every code
      // (round half to even) fits in int16 and code * scale is the value to
      // within half a scale step.  The eight fragments' maxima go through
      // the lane reduction side by side.
      int16_t* P = reinterpret_cast<int16_t*>(p.C_states) + ((size_t)bh * SL + entry - p.c_lo) * DK * DV;
      float* Sc = p.C_scales + ((size_t)bh * SL + entry - p.c_lo) * (DK / 16) * NB;
      float amax[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int rb = j >> 2, cb = (j >> 1) & 1, half = j & 1;
        float a = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(acc[rb][cb][8 * half + e]));
        amax[j] = a;
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1)
#pragma unroll
        for (int j = 0; j < 8; ++j) amax[j] = fmaxf(amax[j], __shfl_xor(amax[j], off, 64));
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int rb = j >> 2, cb = (j >> 1) & 1, half = j & 1;
        const int kblk = (kt * TK + wr0 + 32 * rb) / 32;
        const int nb = (wc0 + 32 * cb) / 32;
        // scale 2^(e - 14) with e the exponent of amax (1 + 2^-15): then
        // amax / scale < 2^15 / (1 + 2^-15), so every code rounds into
        // [-32767, 32767]; both powers of two are built from their exponent
        // fields.  Blocks below 2^-112 (zero or subnormal) take scale 1 and
        // code 0.
        const int E = (int)((__float_as_uint(amax[j] * 1.000030517578125f) >> 23) & 0xffu);
        const bool tiny = E < 15;
        const float inv = tiny ? 1.0f : __uint_as_float((uint32_t)(268 - E) << 23);
        const float sc = tiny ? 1.0f : __uint_as_float((uint32_t)(E - 14) << 23);
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c0 = (int)rintf(acc[rb][cb][8 * half + 2 * q] * inv);
          const int c1 = (int)rintf(acc[rb][cb][8 * half + 2 * q + 1] * inv);
          w[q] = ((uint32_t)c0 & 0xffffu) | ((uint32_t)c1 << 16);
        }
        const int f = (2 * kblk + half) * NB + nb;
        u32x4_t* d = reinterpret_cast<u32x4_t*>(P + (size_t)f * 512 + lane * 8);
        if (p.nt_states) __builtin_nontemporal_store(u32x4_t{w[0], w[1], w[2], w[3]}, d);
        else *d = u32x4_t{w[0], w[1], w[2], w[3]};
        if (lane == 0) Sc[f] = sc;
      }
    }
    uint16_t* P = reinterpret_cast<uint16_t*>(p.C_states) + ((size_t)bh * SL + entry - p.c_lo) * DK * DV * 2;
#pragma unroll
    for (int rb = 0; rb < 2 && !PLAIN && !CODES; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int kblk = (kt * TK + wr0 + 32 * rb) / 32;
        const int nb = (wc0 + 32 * cb) / 32;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          uint32_t hi[4], lo[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            split_bf16x2(acc[rb][cb][8 * half + 2 * e], acc[rb][cb][8 * half + 2 * e + 1], hi[e], lo[e]);
          const size_t blk = ((size_t)(2 * kblk + half) * NB + nb) * 2;
          u32x4_t* dh = reinterpret_cast<u32x4_t*>(P + (blk + 0) * 512 + lane * 8);
          u32x4_t* dl = reinterpret_cast<u32x4_t*>(P + (blk + 1) * 512 + lane * 8);
          if (p.nt_states) {
            // streaming stores: the states are read back by the next kernel,
            // long after they would have left L2
            __builtin_nontemporal_store(u32x4_t{hi[0], hi[1], hi[2], hi[3]}, dh);
            __builtin_nontemporal_store(u32x4_t{lo[0], lo[1], lo[2], lo[3]}, dl);
          } else {
            // plain stores: a block of chunk states is read back right away,
            // from the Infinity Cache
            *dh = u32x4_t{hi[0], hi[1], hi[2], hi[3]};
            *dl = u32x4_t{lo[0], lo[1], lo[2], lo[3]};
          }
        }
      }
    if (!SIG && kt == 0 && tid == 0) {
      if (seg == 0) p.m_states[(size_t)bh * SL + entry - p.c_lo] = M2 * kLn2;
      if (segmented) p.m_local[(size_t)bh * (Nc + 1) + entry] = M2;
    }
  };
  if (seg == 0) {
    write_state(p.c_lo, Mst2);
    if (!SIG && tid < TK) p.n_states[((size_t)bh * SL) * DK + kt * TK + tid] = nreg;
  }

  // flattened block sequence over this segment: block gi covers steps
  // [tb, tb + TB) of chunk c_beg + gi / BPC (BPC = L / TB is a power of two)
  const int BPC = L / TB;
  const int lbpc = 31 - __builtin_clz(BPC);
  const int NBLK = c_end > c_beg ? (c_end - c_beg - 1) * BPC + (min(L, S - (c_end - 1) * L) + TB - 1) / TB : 0;

  // two register sets of loads in flight
  KVec kr[2];
  float ur[2], g2r[2], pmr[2];
  uint4 vr[2][VPT];
  // K, V and the input terms of this head through buffer resources: rows past
  // the end of the sequence read as zero and get weight zero.  Only the last
  // chunk can be short, so that bound is also the chunk's.  The block's first
  // row moves each resource's base and the steps inside the block are in the
  // lane offset (the range check does not see a scalar offset).
  const uint32_t kext = (uint32_t)(((size_t)S * DK - kt * TK) * 2);
  const uint32_t vext = (uint32_t)((size_t)S * DV * 2);
  const uint32_t uext = (uint32_t)((size_t)S * 4);
  const int kvoff = (krs * DK + kcs) * 2;
  const int vvoff = ((tid / VSEG) * DV + (tid % VSEG) * 8) * 2;
  auto load_blk = [&](auto set, int gi) {
    constexpr int s = decltype(set)::value;
    const int c = c_beg + (gi >> lbpc), tb = (gi & (BPC - 1)) * TB;
    const int t0 = c * L, Lc = min(L, S - t0);
    const int trow = t0 + tb;  // first time row of the block
    const __amdgpu_buffer_rsrc_t rk = make_rsrc_at(K, kext, trow * DK * 2);
    if constexpr (EPT == 4) {
      const v2i32_t k2 = __builtin_amdgcn_raw_buffer_load_b64(rk, kvoff, 0, 0);
      kr[s] = make_uint2((uint32_t)k2.x, (uint32_t)k2.y);
    } else {
      kr[s] = buf_load16_nt(rk, kvoff);
    }
    ur[s] = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc_at(p.gu2 + gbase, uext, trow * 4), krs * 4, 0, 0));
    const __amdgpu_buffer_rsrc_t rv = make_rsrc_at(V, vext, trow * DV * 2);
#pragma unroll
    for (int i = 0; i < VPT; ++i) vr[s][i] = buf_load16(rv, vvoff + i * (NT / VSEG) * DV * 2);
    if (tb == 0) {
      g2r[s] = p.gb2[gbase + t0 + Lc - 1];
      pmr[s] = SIG ? 0.0f : p.gpm2[gbase + t0 + Lc - 1];
    }
  };

  // staging side: scalars of the chunk being staged, n partial sums
  float g2s = 0.0f, Mn2s = 0.0f, dec_s = 1.0f;
  float dec_pend = 1.0f, M_pend = 0.0f;   // handed to the matrix-core side
  float np[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) np[e] = 0.0f;
  bool n_pend = false;
  float n_dec = 1.0f;

  // n' = decay n + sum_t w_t k_t: reduce the partial sums over the lanes that
  // share key columns, then (after a barrier) over the waves
  auto flush_n = [&]() {
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      np[e] += __shfl_xor(np[e], 16, 64);
      np[e] += __shfl_xor(np[e], 32, 64);
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
  auto finish_n = [&](int entry) {
    if (tid < TK) {
      float sacc = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) sacc += s_np[w][tid];
      nreg = nreg * n_dec + sacc;
      p.n_states[((size_t)bh * SL + entry - p.c_lo) * DK + kt * TK + tid] = nreg;
    }
    n_pend = false;
  };

  auto stage_blk = [&](auto set, int gi) {
    constexpr int s = decltype(set)::value;
    const int c = c_beg + (gi >> lbpc), tb = (gi & (BPC - 1)) * TB;
    if (tb == 0) {
      if (!SIG && c > c_beg) flush_n();
      const float g2 = g2r[s];
      float Mn2 = 0.0f, dec;
      if constexpr (SIG) {
        dec = exp2f(g2);
      } else {
        Mn2 = g2 + fmaxf(Mst2, pmr[s]);
        dec = exp2f(g2 + Mst2 - Mn2);
        Mst2 = Mn2;
      }
      g2s = g2;
      Mn2s = Mn2;
      dec_s = dec;
      dec_pend = dec;
      M_pend = Mn2;
    }
    // weight 0 for rows past the end of the sequence (zero keys; never inf * 0)
    const float w = c * L + tb + krs < S ? exp2f(g2s + ur[s] - Mn2s) : 0.0f;
    uint16_t* kh = s_kh + s * KBUF + krs * LDK + kcs;
    uint16_t* kl = s_kl + (SPLIT ? s * KBUF + krs * LDK + kcs : 0);
    uint32_t ww[EPT / 2];
    __builtin_memcpy(ww, &kr[s], sizeof(ww));
    uint32_t hi[EPT / 2], lo[EPT / 2];
#pragma unroll
    for (int e = 0; e < EPT / 2; ++e) {
      const float x0 = __uint_as_float(ww[e] << 16) * w;
      const float x1 = __uint_as_float(ww[e] & 0xffff0000u) * w;
      np[2 * e] += x0;
      np[2 * e + 1] += x1;
      if constexpr (SPLIT) split_bf16x2(x0, x1, hi[e], lo[e]);
      else hi[e] = round_bf16x2(x0, x1);
    }
    if constexpr (EPT == 4) {
      *reinterpret_cast<uint2*>(kh) = make_uint2(hi[0], hi[1]);
      if constexpr (SPLIT) *reinterpret_cast<uint2*>(kl) = make_uint2(lo[0], lo[1]);
    } else {
      *reinterpret_cast<uint4*>(kh) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      if constexpr (SPLIT) *reinterpret_cast<uint4*>(kl) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int idx = tid + i * NT;
      const int r = idx / VSEG, sg = idx % VSEG;
      *reinterpret_cast<uint4*>(s_v + s * VBUF + r * LDV + sg * 8) = vr[s][i];
    }
  };

  // matrix-core side
  float M_mma = Mst2;
  auto mma_blk = [&](auto set, int gi) {
    constexpr int s = decltype(set)::value;
    const int c = c_beg + (gi >> lbpc), tb = (gi & (BPC - 1)) * TB;
    if (tb == 0) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) acc[rb][cb] *= dec_pend;
      M_mma = M_pend;
    }
    const int Lc = min(L, S - c * L);
#pragma unroll
    for (int ks = 0; ks < TB / 16; ++ks) {
      if (tb + 16 * ks >= Lc) break;  // uniform: padding only
      bf16x8_t ah[2], al[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        ah[rb] = as_bf16x8(frag_tr_u(s_kh + s * KBUF, LDK, 16 * ks, wr0 + 32 * rb, lane));
        if constexpr (SPLIT) al[rb] = as_bf16x8(frag_tr_u(s_kl + s * KBUF, LDK, 16 * ks, wr0 + 32 * rb, lane));
      }
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const bf16x8_t bv = as_bf16x8(frag_tr_u(s_v + s * VBUF, LDV, 16 * ks, wc0 + 32 * cb, lane));
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          acc[rb][cb] = mma32b(ah[rb], bv, acc[rb][cb]);
          if constexpr (SPLIT) acc[rb][cb] = mma32b(al[rb], bv, acc[rb][cb]);
        }
      }
    }
    if (((gi + 1) & (BPC - 1)) == 0 || gi + 1 == NBLK) write_state(c + 1, M_mma);
  };

  auto iter = [&](auto par, int gi) {
    constexpr int P = decltype(par)::value;
    constexpr int Q = 1 - P;
    if (n_pend) finish_n(c_beg + (gi >> lbpc));
    mma_blk(std::integral_constant<int, P>{}, gi);
    if (gi + 1 < NBLK) stage_blk(std::integral_constant<int, Q>{}, gi + 1);
    if (gi + 3 < NBLK) load_blk(std::integral_constant<int, Q>{}, gi + 3);
    __syncthreads();
  };

  if (NBLK > 0) {
    load_blk(std::integral_constant<int, 0>{}, 0);
    if (NBLK > 1) load_blk(std::integral_constant<int, 1>{}, 1);
    stage_blk(std::integral_constant<int, 0>{}, 0);
    if (NBLK > 2) load_blk(std::integral_constant<int, 0>{}, 2);
    __syncthreads();
    for (int gi = 0; gi < NBLK; gi += 2) {
      iter(std::integral_constant<int, 0>{}, gi);
      if (gi + 1 < NBLK) iter(std::integral_constant<int, 1>{}, gi + 1);
    }
    if constexpr (!SIG) {
      flush_n();
      __syncthreads();
      finish_n(c_end);
    }
  }
  if (segmented) return;  // the join kernels write the final state

  if (p.C_out) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int krow = kt * TK + wr0 + 32 * rb + 8 * (r >> 2) + 4 * h2 + (r & 3);
          const int vcol = wc0 + 32 * cb + l32;
          p.C_out[(size_t)bh * DK * DV + (size_t)krow * DV + vcol] = acc[rb][cb][r];
        }
  }
  if (!SIG && p.n_out && tid < TK) p.n_out[(size_t)bh * DK + kt * TK + tid] = nreg;
  if (!SIG && p.m_out && kt == 0 && tid == 0) p.m_out[bh] = Mst2 * kLn2;
}

// ---- joining sequence segments
//
// A segment s >= 1 ran from a zero state, so its chunk states are local:
// (C_L, n_L) with stabiliser M_L.  With (C_E, n_E, M_E) the true state at the
// segment start and G the summed log-forget gates from there (all in log2
// units), the recurrence being linear in (C, n) with a max-plus stabiliser,
//   M = max(M_L, M_E + G),  C = C_L 2^{M_L - M} + C_E 2^{M_E + G - M}
// (n likewise; sigmoid gate: C = C_L + 2^{G} C_E).  One thread owns 8 packed
// values (one lane slot of a 32 x 32 block, hi and lo planes) of one head,
// and threads with g < DK also own n[g].

struct JoinView {
  uint16_t* st;        // packed states of the head
  const float* nst;    // n states of the head (exp gate)
  size_t stride;       // elements per packed state (hi and lo planes)
  size_t hi;           // element offset of this thread's hi slots
};

__device__ __forceinline__ void join_load(const JoinView& v, int entry, float (&x)[8]) {
  const uint16_t* q = v.st + (size_t)entry * v.stride + v.hi;
  const uint4 h = *reinterpret_cast<const uint4*>(q);
  const uint4 l = *reinterpret_cast<const uint4*>(q + 512);
  const uint32_t hw[4] = {h.x, h.y, h.z, h.w}, lw[4] = {l.x, l.y, l.z, l.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = __uint_as_float(hw[e] << 16) + __uint_as_float(lw[e] << 16);
    x[2 * e + 1] = __uint_as_float(hw[e] & 0xffff0000u) + __uint_as_float(lw[e] & 0xffff0000u);
  }
}

__device__ __forceinline__ void join_store(const JoinView& v, int entry, const float (&x)[8]) {
  uint16_t* q = v.st + (size_t)entry * v.stride + v.hi;
  uint32_t hi[4], lo[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) split_bf16x2(x[2 * e], x[2 * e + 1], hi[e], lo[e]);
  *reinterpret_cast<uint4*>(q) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
  *reinterpret_cast<uint4*>(q + 512) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
}

// Summed log2 forget gates of chunks [c0, c1).
__device__ __forceinline__ float gate_sum2(const StatesParams& p, int bh, int c0, int c1) {
  float g = 0.0f;
  for (int c = c0; c < c1; ++c) g += p.gb2[(size_t)bh * p.S + min((c + 1) * p.L, p.S) - 1];
  return g;
}

// Segment boundaries, in order: the true state at the end of every segment
// (it is the start of the next), and the final state outputs.
template <bool SIG>
__global__ __launch_bounds__(256) void states_carry_kernel(const StatesParams p) {
  const int per = p.DK * p.DV / 8;
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (long long)p.BH * per) return;
  const int bh = (int)(gid / per), g = (int)(gid % per);
  const int Nc = p.Nc;
  JoinView v;
  v.stride = (size_t)p.DK * p.DV * 2;
  v.st = reinterpret_cast<uint16_t*>(p.C_states) + (size_t)bh * (Nc + 1) * v.stride;
  v.nst = SIG ? nullptr : p.n_states + (size_t)bh * (Nc + 1) * p.DK;
  v.hi = (size_t)(g >> 6) * 1024 + (g & 63) * 8;
  const bool own_n = !SIG && g < p.DK;
  const float* ml = p.m_local + (size_t)bh * (Nc + 1);

  float E[8], En = 0.0f, ME2 = 0.0f;
  join_load(v, p.cps, E);  // end of segment 0: already true
  if (own_n) En = v.nst[(size_t)p.cps * p.DK + g];
  if constexpr (!SIG) ME2 = ml[p.cps];
  for (int s = 1; s < p.nseg; ++s) {
    const int c0 = s * p.cps, c1 = min(Nc, c0 + p.cps);
    const float G2 = gate_sum2(p, bh, c0, c1);
    float a = 1.0f, b, MT2 = 0.0f;
    if constexpr (SIG) {
      b = exp2f(G2);
    } else {
      const float ML2 = ml[c1];
      MT2 = fmaxf(ML2, ME2 + G2);
      a = exp2f(ML2 - MT2);
      b = exp2f(ME2 + G2 - MT2);
    }
    float Lv[8];
    join_load(v, c1, Lv);
#pragma unroll
    for (int e = 0; e < 8; ++e) E[e] = Lv[e] * a + E[e] * b;
    join_store(v, c1, E);
    if (own_n) {
      En = v.nst[(size_t)c1 * p.DK + g] * a + En * b;
      p.n_states[((size_t)bh * (Nc + 1) + c1) * p.DK + g] = En;
    }
    if constexpr (!SIG) {
      ME2 = MT2;
      if (g == 0) p.m_states[(size_t)bh * (Nc + 1) + c1] = MT2 * kLn2;
    }
  }
  if (p.C_out) {
    const int blk = g >> 6, ln = g & 63;
    const int kk = blk / (p.DV / 32), nb = blk % (p.DV / 32), h = ln >> 5;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = 16 * kk + (e < 4 ? 4 * h + e : 8 + 4 * h + (e - 4));
      p.C_out[((size_t)bh * p.DK + k) * p.DV + 32 * nb + (ln & 31)] = E[e];
    }
  }
  if (own_n && p.n_out) p.n_out[(size_t)bh * p.DK + g] = En;
  if (!SIG && g == 0 && p.m_out) p.m_out[bh] = ME2 * kLn2;
}

// Interior chunk states of every segment s >= 1 from the true state at the
// segment start (fixed by states_carry_kernel): one thread per (head,
// segment, 8 packed values), which reads the start once and walks up the
// segment's entries with the running gate sum.
template <bool SIG>
__global__ __launch_bounds__(256) void states_fix_kernel(const StatesParams p) {
  const int per = p.DK * p.DV / 8;
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (long long)p.BH * per * (p.nseg - 1)) return;
  const int g = (int)(gid % per);
  const long long rest = gid / per;
  const int s = 1 + (int)(rest % (p.nseg - 1));
  const int bh = (int)(rest / (p.nseg - 1));
  const int Nc = p.Nc;
  const int c0 = s * p.cps, c1 = min(Nc, c0 + p.cps);
  JoinView v;
  v.stride = (size_t)p.DK * p.DV * 2;
  v.st = reinterpret_cast<uint16_t*>(p.C_states) + (size_t)bh * (Nc + 1) * v.stride;
  v.nst = SIG ? nullptr : p.n_states + (size_t)bh * (Nc + 1) * p.DK;
  v.hi = (size_t)(g >> 6) * 1024 + (g & 63) * 8;
  const bool own_n = !SIG && g < p.DK;
  float E[8];
  join_load(v, c0, E);
  const float En = own_n ? v.nst[(size_t)c0 * p.DK + g] : 0.0f;
  // the true stabiliser at the segment start (entry c0 ends the previous
  // segment; segment 0 or states_carry_kernel wrote its true value)
  const float MEt2 = SIG ? 0.0f : p.m_states[(size_t)bh * (Nc + 1) + c0] * kLog2e;
  float G2 = 0.0f;  // summed log2 forget gates of chunks [c0, entry)
  for (int entry = c0 + 1; entry < c1; ++entry) {
    G2 += p.gb2[(size_t)bh * p.S + min(entry * p.L, p.S) - 1];
    float a = 1.0f, b, MT2 = 0.0f;
    if constexpr (SIG) {
      b = exp2f(G2);
    } else {
      const float ML2 = p.m_local[(size_t)bh * (Nc + 1) + entry];
      MT2 = fmaxf(ML2, MEt2 + G2);
      a = exp2f(ML2 - MT2);
      b = exp2f(MEt2 + G2 - MT2);
    }
    float Lv[8];
    join_load(v, entry, Lv);
#pragma unroll
    for (int e = 0; e < 8; ++e) Lv[e] = Lv[e] * a + E[e] * b;
    join_store(v, entry, Lv);
    if (own_n) {
      float* n = p.n_states + ((size_t)bh * (Nc + 1) + entry) * p.DK + g;
      *n = *n * a + En * b;
    }
    if (!SIG && g == 0) p.m_states[(size_t)bh * (Nc + 1) + entry] = MT2 * kLn2;
  }
}

template <int TK, int TV, bool SIG, bool SPLIT, bool PLAIN = false, bool CODES = false>
hipError_t launch_rows(const StatesParams& p, hipStream_t stream) {
  dim3 grid((unsigned)(p.BH * (p.DK / TK) * p.nseg));
  hipLaunchKernelGGL((states_rows_kernel<TK, TV, SIG, SPLIT, PLAIN, CODES>), grid, dim3(512), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nseg <= 1) return e;
  const long long per = (long long)p.BH * (p.DK * p.DV / 8);
  hipLaunchKernelGGL((states_carry_kernel<SIG>), dim3((unsigned)((per + 255) / 256)), dim3(256), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess || p.cps < 2) return e;
  const long long nfix = per * (p.nseg - 1);
  hipLaunchKernelGGL((states_fix_kernel<SIG>), dim3((unsigned)((nfix + 255) / 256)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int TK, int TV>
hipError_t launch_rows_any(const StatesParams& p, bool sig, bool split, hipStream_t stream) {
  if (p.C_scales) {  // int16 codes: one segment, split operands
    if (p.nseg != 1 || p.C_plain || !split) return hipErrorInvalidValue;
    return sig ? launch_rows<TK, TV, true, true, false, true>(p, stream)
               : launch_rows<TK, TV, false, true, false, true>(p, stream);
  }
  if (p.C_plain)  // float32 states only: one segment, split operands
    return sig ? launch_rows<TK, TV, true, true, true>(p, stream) : launch_rows<TK, TV, false, true, true>(p, stream);
  if (sig) return split ? launch_rows<TK, TV, true, true>(p, stream) : launch_rows<TK, TV, true, false>(p, stream);
  return split ? launch_rows<TK, TV, false, true>(p, stream) : launch_rows<TK, TV, false, false>(p, stream);
}

template <int T, bool SIG, bool SPLIT>
hipError_t launch_t(const StatesParams& p, hipStream_t stream) {
  dim3 grid((unsigned)(p.BH * (p.DK / T) * (p.DV / T)));
  hipLaunchKernelGGL((states_wide_kernel<T, T, SIG, SPLIT>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

int rows_tile_rows(int DK, int DV) { return DV == 512 ? 64 : (DV == 256 && DK % 128 == 0 ? 128 : 0); }

hipError_t launch_states_rows_range(const StatesParams& p, bool sig, bool split, hipStream_t stream) {
  StatesParams q = p;
  q.nseg = 1;
  q.cps = (p.c_hi < 0 ? p.Nc : p.c_hi) - p.c_lo;
  q.C_plain = nullptr;
  q.plain_only = 0;
  q.m_local = nullptr;
  const int tk = rows_tile_rows(p.DK, p.DV);
  if (tk == 64) return launch_rows_any<64, 512>(q, sig, split, stream);
  if (tk == 128) return launch_rows_any<128, 256>(q, sig, split, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_states_wide(const StatesParams& p, bool sig, bool split, hipStream_t stream) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  // Whole-row tiles (TK x DV) when they still give every CU a workgroup.
  // Whole-row tiles; with too few heads to fill the CUs the sequence is cut
  // into segments that run at once and are joined afterwards.
  const int rows_tk = rows_tile_rows(p.DK, p.DV);
  if (p.C_scales) {
    // int16 codes: the row-tile kernel in one segment (the joins work on the
    // hi + lo form)
    if (!rows_tk || p.C_plain) return hipErrorInvalidValue;
    StatesParams q = p;
    q.nseg = 1;
    q.cps = p.Nc;
    return rows_tk == 64 ? launch_rows_any<64, 512>(q, sig, split, stream)
                         : launch_rows_any<128, 256>(q, sig, split, stream);
  }
  if (rows_tk) {
    StatesParams q = p;
    const long long base = (long long)p.BH * (p.DK / rows_tk);
    q.nseg = 1;
    q.cps = p.Nc;
    if (base < cus && p.Nc >= 2 && p.m_local) {
      const long long want = (cus + base - 1) / base;
      q.cps = (int)((p.Nc + want - 1) / want);
      q.nseg = (p.Nc + q.cps - 1) / q.cps;
    }
    if (base >= cus || q.nseg > 1) {
      // segment-local states are joined afterwards: the plain copy then
      // comes from the joined packed states
      if (q.nseg > 1 || !split || !q.plain_only) {
        q.C_plain = nullptr;
        q.plain_only = 0;
      }
      hipError_t e = rows_tk == 64 ? launch_rows_any<64, 512>(q, sig, split, stream)
                                   : launch_rows_any<128, 256>(q, sig, split, stream);
      if (e == hipSuccess && p.C_plain && !q.C_plain)
        e = launch_unpack_states(p.C_states, p.C_plain, (long long)p.BH * (p.Nc + 1), p.DK, p.DV, stream);
      return e;
    }
  }
  if (p.C_plain) {
    StatesParams q = p;
    q.C_plain = nullptr;
    q.plain_only = 0;
    hipError_t e = launch_states_wide(q, sig, split, stream);
    if (e == hipSuccess)
      e = launch_unpack_states(p.C_states, p.C_plain, (long long)p.BH * (p.Nc + 1), p.DK, p.DV, stream);
    return e;
  }
  // 128-wide tiles when they still give at least two workgroups per CU.
  const bool big = (long long)p.BH * (p.DK / 128) * (p.DV / 128) >= 2LL * cus;
  if (big) {
    if (sig) return split ? launch_t<128, true, true>(p, stream) : launch_t<128, true, false>(p, stream);
    return split ? launch_t<128, false, true>(p, stream) : launch_t<128, false, false>(p, stream);
  }
  if (sig) return split ? launch_t<64, true, true>(p, stream) : launch_t<64, true, false>(p, stream);
  return split ? launch_t<64, false, true>(p, stream) : launch_t<64, false, false>(p, stream);
}

}  // namespace mlstm
