// Fused chunk walker (gfx950): the whole chunkwise forward pass in one launch,
// with the chunk states kept in registers instead of being written out and
// read back between two kernels.
//
// The chunkwise form ("Tiled Flash Linear Attention: More Efficient Linear RNN
// and xLSTM Kernels", abstract: an inter-chunk recurrence plus a parallel
// intra-chunk part with a second level of sequence tiling; the mLSTM cell of
// "xLSTM: the NX-AI repository behind the extended LSTM architecture",
// section "Exponential gating, matrix memory, and why the kernels decide
// everything") computes, for chunk c of a head,
//   H_c = (inter term Q_c C_{c-1}, rows scaled) + (causal, gate-decayed
//         Q_c K_c^T) V_c, then the normaliser division (exp gate),
//   C_c = decay C_{c-1} + K_c^T (w . V_c)       w = per-step gate weights.
// The TFLA page lists avoiding the HBM round trip of those per-chunk states
// as a planned follow-up; this kernel is that fused form.
//
// Organisation.  One workgroup (8 waves, two per SIMD) owns one head and a
// 128-column slice of V / H / C and walks the chunks of the head in order.
// The waves split by role, so that the two waves sharing a SIMD run
// different instruction mixes and overlap instead of moving through the same
// phases in step:
//   intra waves 0..3   wave a owns queries 16 a .. 16 a + 15 of every 64-row
//                      query tile and all 128 columns of their H rows.  Per
//                      32-key tile it forms S^T = K Q^T on 16x16x32 MFMAs,
//                      P = s S decay in registers, and H += P V straight from
//                      those registers (the score accumulators already have
//                      the layout of the P.V operand, with the keys taken in a
//                      permuted order that the V reads follow).  These waves
//                      also stage every Q, K and V tile and form the gate
//                      terms of each chunk from the raw gate inputs.
//   state waves 4..7   wave 4 + b holds the state block C[0 .. DK-1][32 b ..
//                      32 b + 31] for the whole walk, forms the inter term
//                      Q C for its columns at the start of every query tile
//                      (handed to the intra waves through LDS) and, on the
//                      last query tile of a chunk, the update
//                      C = decay C + K^T (w . V) from the same key tiles.
// Each role runs its own loop nest; both pass the same workgroup barriers in
// the same order: one per chunk for the gate terms [G], one per query tile
// for Q [Q], one per key tile [R] and one at the end of the chunk [N].
//
// Gate terms.  With lf = log sigmoid(f) and i~ = i (exp gate) or
// log sigmoid(i) (sig gate), the chunk needs, in log2 units, the in-chunk
// inclusive sums b_t = lf_0 + ... + lf_t, u_t = i~_t - b_t and (exp gate)
// the running maximum pm_t = max(u_0 .. u_t).  Before [G] each intra wave
// scans its 64-position segments (positions 64 s .. 64 s + 63 of the chunk,
// s = 4 e + wave) with lane shuffles and posts the segment's sum and the
// maximum of its local u; after [G] each thread adds the sums of the earlier
// segments to its own positions (u moves down by the same amount, the running
// maximum takes the earlier segments' maxima) and the finished terms are read
// after [Q].  No separate pass or workspace is needed.  The
// four column slices of a head compute the same score tiles (the price of
// keeping C on-chip); they are placed on one XCD so their Q and K reads share
// an L2.
//
// Precision.  P, the state and w . V enter the matrix cores as bf16 hi + lo
// pairs (about 16 significant bits, two MFMA passes); Q, K and V enter
// unchanged.  Between chunks a state wave holds its block in that split form;
// the last query tile of a chunk rebuilds float32 accumulators from it,
// applies the decay, accumulates the update and splits again, so the state is
// rounded to 16 significant bits once per chunk (relative 2^-17; the decay
// keeps it from growing).
//
// Contraction order of the state.  Accumulator row m of each 32-row block
// holds k index perm(m) (4-row groups 1 and 2 of every 16 swapped); the K^T
// operand of the update is read with that permutation, so the values a lane
// holds for a 16-deep k step of Q C are the k indices 8 (lane / 32) + e in
// natural order and Q enters with plain 16-byte row reads.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "pair_store.h"

namespace mlstm {
namespace {

constexpr int kWalkMaxL = 512;
constexpr int kWalkSlice = 128;

// K and V tile rows are stored unpadded with their 16-byte column groups
// XOR-swizzled by row (period 16 rows): the 16-byte row reads (16
// consecutive rows, one group) and the transposing reads (4 or 16
// consecutive rows, 2 or 4 consecutive groups) then fall on distinct banks.
__device__ __forceinline__ int kswz(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }

// element offset of (row r, column c) in a swizzled tile with rows of W elements
template <int W>
__device__ __forceinline__ int swz(int r, int c) {
  return r * W + (((c >> 3) ^ kswz(r)) << 3) + (c & 7);
}

// For a fixed row r, the columns 32 x + c0 (c0 < 32 a multiple of 4) of a
// row of W elements sit at base(x & 3) + 128 (x >> 2): the swizzle permutes
// the four 32-column blocks of every 128 columns among themselves, so the
// four bases below and immediate offsets cover a whole row.
template <int W>
__device__ __forceinline__ int swz_base(int r, int c0, int x) {
  const int k = kswz(r);
  return r * W + 32 * (x ^ (k >> 2)) + 8 * (((c0 >> 3) ^ k) & 3) + (c0 & 7);
}

// Inclusive scan (sum or max) over the 64 lanes of a wave.
template <bool IS_MAX>
__device__ __forceinline__ float wave_scan(float x) {
  const int lane = (int)threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(x, off, 64);
    if (lane >= off) x = scan_op<IS_MAX>(x, y);
  }
  return x;
}

__device__ __forceinline__ uint2 lds_tr(const uint16_t* p) {
  const short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)(p));
  return __builtin_bit_cast(uint2, v);
}

template <int DK, bool SIG>
__global__ __launch_bounds__(512) void walk_kernel(const WalkParams p) {
  constexpr int NA = 256;                  // threads of the intra role
  constexpr int TQ = 64, TKV = 32, TVS = kWalkSlice;
  constexpr int LDQ = DK + 8;              // 16-byte row reads: 4 banks mod 64
  constexpr int NKB = DK / 32;             // 32-row state blocks of a state wave
  constexpr int NKS = DK / 16;             // 16-deep k steps of Q C
  constexpr int NSS = DK / 32;             // 32-deep k steps of the scores
  constexpr int KG = DK / 8;               // 16-byte groups per Q / K row
  constexpr int VG = TVS / 8;              // per V row
  constexpr int QPT = TQ * KG / NA;        // Q pieces per staging thread
  constexpr int KPT = TKV * KG / NA;       // K pieces
  constexpr int VPT = TKV * VG / NA;       // V pieces
  constexpr int NCB = TVS / 16;            // 16-column blocks of an intra wave's H rows
  constexpr int LDX = TQ + 4;              // inter term, stored [column][row]
  constexpr int GPT = kWalkMaxL / NA;      // gate positions per staging thread
  static_assert(QPT * NA == TQ * KG && KPT * NA == TKV * KG && VPT * NA == TKV * VG, "staging split");
  static_assert(DK <= NA && KG == 32, "one state-role thread per normaliser entry; 32 column groups");

  __shared__ __align__(16) uint16_t s_q[TQ * LDQ];
  __shared__ __align__(16) uint16_t s_kb[2][TKV * DK];   // K tiles, double buffered
  __shared__ __align__(16) uint16_t s_vb[2][TKV * TVS];  // V tiles, double buffered
  __shared__ __align__(16) float s_xt[TVS * LDX];        // inter term of the query tile
  __shared__ __align__(16) float s_gu[kWalkMaxL];
  __shared__ __align__(16) float s_gb[kWalkMaxL];
  __shared__ __align__(16) float s_gpm[SIG ? 4 : kWalkMaxL];
  __shared__ float s_segT[kWalkMaxL / 64], s_segX[kWalkMaxL / 64];  // per-segment sum of lf, max of local u
  __shared__ __align__(16) uint16_t s_nh[DK], s_nl[DK];  // normaliser as bf16 hi / lo
  __shared__ __align__(16) float s_np[SIG ? 4 : 4 * DK];

  const int S = p.S, L = p.L, Nc = p.Nc, DV = p.DV;
  const int NS = DV / TVS;
  // workgroup -> (head, slice); with BH a multiple of 8 the slices of one
  // head share blockIdx % 8, i.e. one XCD
  int slice, bh;
  {
    const int bid = blockIdx.x;
    if ((p.BH & 7) == 0) {
      const int x = bid & 7, jj = bid >> 3;
      slice = jj % NS;
      bh = (jj / NS) * 8 + x;
    } else {
      slice = bid % NS;
      bh = bid / NS;
    }
  }
  const int v0 = slice * TVS;
  const float scale = p.scale;
  const float log2_scale = log2f(p.scale);
  const size_t gbase = (size_t)bh * S;
  const int wave0 = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);

  // chunk geometry, computed alike by both roles
  auto chunk_len = [&](int c) { return min(L, S - c * L); };
  auto nsub_of = [&](int Lc) { return (Lc + TQ - 1) / TQ; };
  auto nkt_of = [&](int Lc, int i) { return min(2 * i + 2, (Lc + TKV - 1) / TKV); };
  // chunk scalars: log2 forget sum g2, stabiliser after the chunk, decay of the old state
  auto chunk_scalars = [&](int Lc, float M, float& g2, float& Mn, float& dec) {
    g2 = s_gb[Lc - 1];
    if constexpr (SIG) {
      Mn = 0.0f;
      dec = exp2f(g2);
    } else {
      Mn = g2 + fmaxf(M, s_gpm[Lc - 1]);
      dec = exp2f(g2 + M - Mn);
    }
  };
  float M = (!SIG && p.m0) ? p.m0[bh] * kLog2e : 0.0f;  // stabiliser, log2 units

  if (wave0 < 4) {
    // =====================================================================
    // intra role
    // =====================================================================
    int tid, lane, wa, l16, g4;
    auto set_roles = [&]() {
      int t = (int)threadIdx.x;
      asm volatile("" : "+v"(t));
      int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
      asm volatile("" : "+s"(w));
      tid = t;
      lane = t & 63;
      wa = w;
      l16 = lane & 15;
      g4 = lane >> 4;
    };
    set_roles();
    const uint16_t* Qh = static_cast<const uint16_t*>(p.Q) + gbase * DK;
    const uint16_t* Kh = static_cast<const uint16_t*>(p.K) + gbase * DK;
    const uint16_t* Vh = static_cast<const uint16_t*>(p.V) + gbase * DV + v0;

    // ---- global loads, one step ahead.  Q tiles in (chunk, query tile)
    // order; K / V tiles in (chunk, query tile, key tile) order.  Piece e of
    // a thread is piece tid + 256 e of the tile (16 bytes, row-major groups).
    uint4 qpre[QPT], kpre[KPT], vpre[VPT];
    float gpre_f[GPT], gpre_i[GPT];
    int qc = 0, qi = 0;          // next Q tile to load
    int kc = 0, ki = 0, kj = 0;  // next K / V tile to load
    auto load_q = [&]() {
      if (qc >= Nc) return;
      const int t0 = qc * L, Lc = chunk_len(qc), r0 = qi * TQ;
      // rows past the chunk read as zero: the load steps are in the lane
      // offset, which the range check covers
      const __amdgpu_buffer_rsrc_t rq = make_rsrc(Qh + (size_t)(t0 + r0) * DK, (uint32_t)((Lc - r0) * DK * 2));
#pragma unroll
      for (int e = 0; e < QPT; ++e) qpre[e] = buf_load16(rq, tid * 16 + e * NA * 16);
      if (++qi >= nsub_of(Lc)) {
        qi = 0;
        ++qc;
      }
    };
    auto load_kv = [&]() {
      if (kc >= Nc) return;
      const int t0 = kc * L, Lc = chunk_len(kc), k0 = kj * TKV;
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kh + (size_t)(t0 + k0) * DK, (uint32_t)((Lc - k0) * DK * 2));
      const __amdgpu_buffer_rsrc_t rv =
          make_rsrc(Vh + (size_t)(t0 + k0) * DV, (uint32_t)(((Lc - k0 - 1) * DV + TVS) * 2));
#pragma unroll
      for (int e = 0; e < KPT; ++e) kpre[e] = buf_load16(rk, tid * 16 + e * NA * 16);
#pragma unroll
      for (int e = 0; e < VPT; ++e)
        vpre[e] = buf_load16(rv, ((tid / VG) * DV + (tid % VG) * 8) * 2 + e * (NA / VG) * DV * 2);
      if (++kj >= nkt_of(Lc, ki)) {
        kj = 0;
        if (++ki >= nsub_of(Lc)) {
          ki = 0;
          ++kc;
        }
      }
    };
    auto load_gates = [&](int c) {
      if (c >= Nc) return;
      const int t0 = c * L, Lc = chunk_len(c);
#pragma unroll
      for (int e = 0; e < GPT; ++e) {
        const int t = tid + e * NA;
        const bool ok = t < Lc;
        gpre_f[e] = ok ? p.f_pre[gbase + t0 + t] : 0.0f;
        gpre_i[e] = ok ? p.i_pre[gbase + t0 + t] : 0.0f;
      }
    };
    // LDS offsets of this thread's K and V pieces (rows tid / 32 + 8 e and
    // tid / 16 + 16 e), fixed for the whole walk
    int kso[KPT], vso[VPT];
#pragma unroll
    for (int e = 0; e < KPT; ++e) kso[e] = swz<DK>((tid + e * NA) / KG, (tid % KG) * 8);
#pragma unroll
    for (int e = 0; e < VPT; ++e) vso[e] = swz<TVS>((tid + e * NA) / VG, (tid % VG) * 8);
    // K / V tile n of the sequence sits in buffer n % 2; stage() writes the
    // tile held in registers into buffer buf and requests the next one.
    bool have_kv = false;
    auto stage = [&](int buf) {
      if (have_kv) {
#pragma unroll
        for (int e = 0; e < KPT; ++e) *reinterpret_cast<uint4*>(s_kb[buf] + kso[e]) = kpre[e];
#pragma unroll
        for (int e = 0; e < VPT; ++e) *reinterpret_cast<uint4*>(s_vb[buf] + vso[e]) = vpre[e];
      }
      have_kv = kc < Nc;
      load_kv();
    };
    load_gates(0);
    load_q();
    have_kv = kc < Nc;
    load_kv();
    stage(0);
    int ks = 0;  // key tiles consumed

    for (int c = 0; c < Nc; ++c) {
      set_roles();
      const int t0 = c * L, Lc = chunk_len(c);
      const int nsub = nsub_of(Lc);
      // segment-local gate terms of this thread's positions; u past the end
      // of a short last chunk is -inf, so those keys (zero rows) get weight
      // exactly zero
      float lb[GPT], lu[GPT], lpm[GPT];
#pragma unroll
      for (int e = 0; e < GPT; ++e) {
        const int t = tid + e * NA;
        const bool ok = t < Lc;
        lb[e] = wave_scan<false>(ok ? log_sigmoid(gpre_f[e]) * kLog2e : 0.0f);
        lu[e] = ok ? (SIG ? log_sigmoid(gpre_i[e]) : gpre_i[e]) * kLog2e - lb[e] : -INFINITY;
        lpm[e] = SIG ? 0.0f : wave_scan<true>(lu[e]);
        if (lane == 63) {
          s_segT[t >> 6] = lb[e];
          s_segX[t >> 6] = lpm[e];
        }
      }
      load_gates(c + 1);
      __syncthreads();  // [G] gate terms
      // add the earlier segments (uniform per wave) to this thread's positions
#pragma unroll
      for (int e = 0; e < GPT; ++e) {
        const int t = tid + e * NA;
        float B = 0.0f, P = -INFINITY;
        for (int sg = 0; sg < (t >> 6); ++sg) {
          if constexpr (!SIG) P = fmaxf(P, s_segX[sg] - B);
          B += s_segT[sg];
        }
        s_gb[t] = lb[e] + B;
        s_gu[t] = lu[e] - B;
        if constexpr (!SIG) s_gpm[t] = fmaxf(P, lpm[e] - B);
      }
      float g2, Mn, dec;  // set after the first [Q] of the chunk
      float np[8];  // n partial sums of this thread's K column group (exp gate)
#pragma unroll
      for (int e = 0; e < 8; ++e) np[e] = 0.0f;

      for (int i = 0; i < nsub; ++i) {
        set_roles();
        const int row0 = i * TQ;
#pragma unroll
        for (int e = 0; e < QPT; ++e) {
          const int idx = tid + e * NA;
          *reinterpret_cast<uint4*>(s_q + (idx / KG) * LDQ + (idx % KG) * 8) = qpre[e];
        }
        load_q();
        __syncthreads();  // [Q] query tile
        set_roles();
        if (i == 0) chunk_scalars(Lc, M, g2, Mn, dec);
        // this wave's 16 queries as B fragments of the 16x16x32 score blocks
        uint4 qf[NSS];
#pragma unroll
        for (int s = 0; s < NSS; ++s)
          qf[s] = *reinterpret_cast<const uint4*>(s_q + (16 * wa + l16) * LDQ + 32 * s + 8 * g4);
        // per-row terms of this lane's query: exponent offset r2 of P (with
        // log2 s; -inf past the chunk end), weight of the inter term (with
        // s), stabiliser m (log2 units)
        float r2 = -INFINITY, wrq = 0.0f, m2q = 0.0f;
        {
          const int tau = row0 + 16 * wa + l16;
          if (tau < Lc) {
            const float b2 = s_gb[tau];
            if constexpr (SIG) {
              r2 = b2 + log2_scale;
              wrq = exp2f(b2) * scale;
            } else {
              const float mx = fmaxf(M, s_gpm[tau]);
              r2 = log2_scale - mx;
              wrq = exp2f(M - mx) * scale;
              m2q = b2 + mx;
            }
          }
        }
        // normaliser contribution of the state, q . n, on the matrix cores:
        // every row of the A operand is n (bf16 hi + lo), so each lane ends
        // with the full sum for its query l16
        float dint = 0.0f;
        if constexpr (!SIG) {
          float4_t dacc[2] = {float4_t{0.0f, 0.0f, 0.0f, 0.0f}, float4_t{0.0f, 0.0f, 0.0f, 0.0f}};
          uint4 nf[NSS][2];
#pragma unroll
          for (int s = 0; s < NSS; ++s) {
            nf[s][0] = *reinterpret_cast<const uint4*>(s_nh + 32 * s + 8 * g4);
            nf[s][1] = *reinterpret_cast<const uint4*>(s_nl + 32 * s + 8 * g4);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int s = 0; s < NSS; ++s) {
            dacc[0] = mma16b(as_bf16x8(nf[s][0]), as_bf16x8(qf[s]), dacc[0]);
            dacc[1] = mma16b(as_bf16x8(nf[s][1]), as_bf16x8(qf[s]), dacc[1]);
          }
          dint = dacc[0][0] + dacc[1][0];
        }
        float4_t hacc[NCB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) hacc[cb] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
        float dpart = 0.0f;

        int kfa[4];  // this lane's K row l16, columns 8 g + 32 x (x < 4)
#pragma unroll
        for (int x = 0; x < 4; ++x) kfa[x] = swz_base<DK>(l16, 8 * g4, x);
        const int nkt = nkt_of(Lc, i);
        for (int j = 0; j < nkt; ++j) {
          const int cur = ks & 1;
          const uint16_t* const s_k = s_kb[cur];
          const uint16_t* const s_v = s_vb[cur];
          const int key0 = j * TKV;
          // 16-key blocks 2j and 2j + 1 of the chunk against this wave's
          // 16-query block 4i + a: below it fully live, equal to it on the
          // diagonal (causal select), above it zero (skipped)
          auto block = [&](auto nlive_c, auto diag_c) {
            constexpr int NLIVE = decltype(nlive_c)::value;
            constexpr bool DIAG = decltype(diag_c)::value;
            float4_t sacc[2][2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
              for (int x = 0; x < 2; ++x) sacc[kb][x] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
            // K reads in two halves of the DK range, each half's reads all out
            // before its MFMAs (a scheduling barrier keeps the compiler from
            // sinking each read to its use)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              uint4 kf[NSS / 2][2];
#pragma unroll
              for (int x = 0; x < NSS / 2; ++x)
#pragma unroll
                for (int kb = 0; kb < NLIVE; ++kb)
                  kf[x][kb] = *reinterpret_cast<const uint4*>(s_k + kfa[x] + 128 * hh + 16 * kb * DK);
              __builtin_amdgcn_sched_barrier(0);
#pragma unroll
              for (int x = 0; x < NSS / 2; ++x)
#pragma unroll
                for (int kb = 0; kb < NLIVE; ++kb)
                  sacc[kb][x & 1] = mma16b(as_bf16x8(kf[x][kb]), as_bf16x8(qf[4 * hh + x]), sacc[kb][x & 1]);
              __builtin_amdgcn_sched_barrier(0);
            }
            // the V reads of the first four column blocks go out next, so that
            // they overlap the forming of P
            const int vb0 = swz<TVS>(4 * g4 + (l16 >> 2), 4 * (l16 & 3));
            constexpr int NCH = NCB / 2;
            uint2 vx[NCH][2];
            auto read_v = [&](int cb0) {
#pragma unroll
              for (int x = 0; x < NCH; ++x) {
                vx[x][0] = lds_tr(s_v + (vb0 ^ ((cb0 + x) << 4)));
                vx[x][1] = lds_tr(s_v + (vb0 ^ ((cb0 + x) << 4)) + 16 * TVS);
              }
            };
            read_v(0);
            __builtin_amdgcn_sched_barrier(0);
            // P for keys key0 + 16 kb + 4 g + e (slot 4 kb + e of the P.V
            // operand) as bf16 hi / lo words; rows past the chunk end have
            // r2 = -inf and keys past it u = -inf, so only the diagonal block
            // needs the causal select
            uint32_t ph[4], pl[4];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
              if (kb >= NLIVE) {
                ph[2 * kb] = ph[2 * kb + 1] = pl[2 * kb] = pl[2 * kb + 1] = 0u;
                continue;
              }
              const float4 u4 = *reinterpret_cast<const float4*>(s_gu + key0 + 16 * kb + 4 * g4);
              const float uu[4] = {u4.x, u4.y, u4.z, u4.w};
              float val[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                val[e] = (sacc[kb][0][e] + sacc[kb][1][e]) * __builtin_amdgcn_exp2f(r2 + uu[e]);
                if (DIAG && kb == NLIVE - 1) val[e] = (4 * g4 + e <= l16) ? val[e] : 0.0f;
                dpart += val[e];
              }
              split_bf16x2(val[0], val[1], ph[2 * kb], pl[2 * kb]);
              split_bf16x2(val[2], val[3], ph[2 * kb + 1], pl[2 * kb + 1]);
            }
            const bf16x8_t ahi = as_bf16x8(make_uint4(ph[0], ph[1], ph[2], ph[3]));
            const bf16x8_t alo = as_bf16x8(make_uint4(pl[0], pl[1], pl[2], pl[3]));
            // V rows in the same key order (slot e < 4: key 4 g + e, slot
            // e >= 4: key 16 + 4 g + e - 4), by transposing reads: lane j of
            // each 16-lane group addresses row 4 g + j / 4 (and 16 rows
            // further), columns 16 cb + 4 (j % 4) ..; the swizzle repeats
            // every 16 rows and moves with cb as an XOR of bits 4..6
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              if (hh) {
                read_v(NCH);
                __builtin_amdgcn_sched_barrier(0);
              }
#pragma unroll
              for (int x = 0; x < NCH; ++x)
                hacc[NCH * hh + x] = mma16b(
                    ahi, as_bf16x8(make_uint4(vx[x][0].x, vx[x][0].y, vx[x][1].x, vx[x][1].y)), hacc[NCH * hh + x]);
#pragma unroll
              for (int x = 0; x < NCH; ++x)
                hacc[NCH * hh + x] = mma16b(
                    alo, as_bf16x8(make_uint4(vx[x][0].x, vx[x][0].y, vx[x][1].x, vx[x][1].y)), hacc[NCH * hh + x]);
            }
          };
          const int qblk = 4 * i + wa;
          if (2 * j + 1 < qblk) block(std::integral_constant<int, 2>{}, std::false_type{});
          else if (2 * j + 1 == qblk) block(std::integral_constant<int, 2>{}, std::true_type{});
          else if (2 * j == qblk) block(std::integral_constant<int, 1>{}, std::true_type{});
          // n partial sums (exp gate) on the last query tile, which visits
          // every key tile of the chunk: this thread's K pieces of the tile,
          // weighted (piece tid + 256 e: row tid / 32 + 8 e, column group tid % 32)
          if (!SIG && i == nsub - 1) {
#pragma unroll
            for (int e = 0; e < KPT; ++e) {
              const int row = tid / KG + e * (NA / KG);
              const float w = __builtin_amdgcn_exp2f(g2 + s_gu[key0 + row] - Mn);
              const uint4 kv = *reinterpret_cast<const uint4*>(s_k + kso[e]);
              const uint32_t kw[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                np[2 * q] += w * __uint_as_float(kw[q] << 16);
                np[2 * q + 1] += w * __uint_as_float(kw[q] & 0xffff0000u);
              }
            }
          }
          // the next tile into the other buffers (last read before the previous barrier)
          stage(cur ^ 1);
          ++ks;
          __syncthreads();  // [R] key tile
        }

        // ---- normaliser, inter term and H for this wave's rows.  After the
        // reductions every lane holds the sums of query l16; lane 4 g + r
        // supplies the values of accumulator row 4 g + r.
        float inv = 1.0f;
        if constexpr (!SIG) {
          dpart += __shfl_xor(dpart, 16, 64);
          dpart += __shfl_xor(dpart, 32, 64);
          const float d = dint * wrq + dpart;
          inv = 1.0f / (fmaxf(fabsf(d), exp2f(-m2q)) + p.eps);
          // per-row m and normaliser for a backward pass, from the first
          // column slice (lanes 0..15 hold queries 0..15 of the wave)
          const int tau = row0 + 16 * wa + l16;
          if (v0 == 0 && g4 == 0 && tau < Lc) {
            if (p.m_rows) p.m_rows[gbase + t0 + tau] = m2q * kLn2;
            if (p.den_rows) p.den_rows[gbase + t0 + tau] = d;
          }
        }
        float iv[4], wv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          iv[r] = SIG ? 1.0f : __shfl(inv, 4 * g4 + r, 64);
          wv[r] = __shfl(wrq, 4 * g4 + r, 64);
        }
        auto store_h = [&](auto esize) {
          constexpr int E = decltype(esize)::value;
          // rows past the chunk fall outside the resource and are dropped (the
          // row and column steps are in the lane offset)
          const __amdgpu_buffer_rsrc_t rh =
              make_rsrc(static_cast<const char*>(p.H) + ((gbase + t0 + row0) * DV + v0) * E,
                        (uint32_t)(((Lc - row0 - 1) * DV + TVS) * E));
          float4 xr[NCB];
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
            xr[cb] = *reinterpret_cast<const float4*>(s_xt + (16 * cb + l16) * LDX + 16 * wa + 4 * g4);
          __builtin_amdgcn_sched_barrier(0);
          // Plain stores: a store instruction covers 64-byte (float32) or
          // 32-byte (bf16) pieces of H rows, which L2 merges into whole lines
          // (with the streaming hint each piece went out on its own and the
          // written bytes grew by half).  float32: one value per lane and
          // store.  bf16: lane pairs (l16 even, odd) swap values so that the
          // even lane holds rows 0 and 2 of its quad and the odd lane rows 1
          // and 3, each as two adjacent columns, rounded together and stored
          // as one word (measured 4-5 % faster than one 2-byte store per value;
          // the same exchange with 8-byte float32 stores was 3-4 % slower).
          const bool odd = (l16 & 1) != 0;
          const int hvoff = E == 2 ? ((16 * wa + 4 * g4 + (odd ? 1 : 0)) * DV + (l16 & ~1)) * E
                                   : ((16 * wa + 4 * g4) * DV + l16) * E;
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) {
            const float xv[4] = {xr[cb].x, xr[cb].y, xr[cb].z, xr[cb].w};
            float hv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) hv[r] = (hacc[cb][r] + wv[r] * xv[r]) * iv[r];
            if constexpr (E == 2) {
#pragma unroll
              for (int rp = 0; rp < 2; ++rp) {
                const float2 pr = pair_rows_to_cols(hv[2 * rp], hv[2 * rp + 1], odd);
                __builtin_amdgcn_raw_buffer_store_b32(round_bf16x2(pr.x, pr.y), rh,
                                                      hvoff + (2 * rp * DV + 16 * cb) * E, 0, 0);
              }
            } else {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(hv[r]), rh, hvoff + (r * DV + 16 * cb) * E, 0, 0);
            }
          }
        };
        if (p.h_bf16) store_h(std::integral_constant<int, 2>{});
        else store_h(std::integral_constant<int, 4>{});
      }
      // lanes l and l + 32 of a wave share a column group; the four waves'
      // partial sums go to LDS for the state role
      if constexpr (!SIG) {
#pragma unroll
        for (int e = 0; e < 8; ++e) np[e] += __shfl_xor(np[e], 32, 64);
        if (lane < KG) {
#pragma unroll
          for (int e = 0; e < 8; ++e) s_np[wa * DK + lane * 8 + e] = np[e];
        }
      }
      __syncthreads();  // [N] end of chunk
      M = Mn;
    }
  } else {
    // =====================================================================
    // state role
    // =====================================================================
    int tid, tb, lane, wb, h, l32;
    auto set_roles = [&]() {
      int t = (int)threadIdx.x;
      asm volatile("" : "+v"(t));
      int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
      asm volatile("" : "+s"(w));
      tid = t;
      tb = t - NA;
      lane = t & 63;
      wb = w - 4;
      h = lane >> 5;
      l32 = lane & 31;
    };
    set_roles();
    auto vcol = [&]() { return v0 + 32 * wb + l32; };  // the state column of this lane
    // Accumulator register r of block kb holds C[dk][vcol] with
    // dk = 32 kb + perm(row of r); chi / clo hold the block as bf16 hi + lo
    // words, word q packing registers 2q (low half) and 2q + 1.
    auto state_row = [&](int kb, int r) {
      const int j = r >> 2;
      return 32 * kb + 16 * (j >> 1) + 8 * h + 4 * (j & 1) + (r & 3);
    };
    uint32_t chi[NKB][8], clo[NKB][8];
    auto split_state = [&](const float16_t* acc) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int q = 0; q < 8; ++q) split_bf16x2(acc[kb][2 * q], acc[kb][2 * q + 1], chi[kb][q], clo[kb][q]);
    };
    auto write_state = [&](const float16_t* acc) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          p.C_out[(size_t)bh * DK * DV + (size_t)state_row(kb, r) * DV + vcol()] = acc[kb][r];
    };
    {
      // a zero-extent resource reads zeros when there is no initial state
      const __amdgpu_buffer_rsrc_t rc =
          make_rsrc(p.C0 ? p.C0 + (size_t)bh * DK * DV : p.f_pre, p.C0 ? (uint32_t)(DK * DV * 4) : 0u);
      float16_t c0[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          c0[kb][r] = __builtin_bit_cast(
              float, __builtin_amdgcn_raw_buffer_load_b32(rc, (state_row(kb, r) * DV + vcol()) * 4, 0, 0));
      if (Nc == 0 && p.C_out) write_state(c0);  // empty sequence: the initial state, exactly
      split_state(c0);
    }
    float nst = 0.0f;  // normaliser entry tb (exp gate), also kept in s_nh / s_nl
    auto put_n = [&]() {
      const uint16_t hi = f32_to_bf16(nst);
      s_nh[tb] = hi;
      s_nl[tb] = f32_to_bf16(nst - __uint_as_float((uint32_t)hi << 16));
    };
    if constexpr (!SIG) {
      nst = p.n0 ? p.n0[(size_t)bh * DK + tb] : 0.0f;
      put_n();
    }
    int ks = 0;  // key tiles consumed

    for (int c = 0; c < Nc; ++c) {
      set_roles();
      const int Lc = chunk_len(c);
      const int nsub = nsub_of(Lc);
      __syncthreads();  // [G] gate terms
      float g2, Mn, dec;  // set after the first [Q] of the chunk
      // query tile i; LAST: the chunk's last tile, which also updates the state
      auto sub_tile = [&](auto last_c, int i) {
        constexpr bool last = decltype(last_c)::value;
        set_roles();
        __syncthreads();  // [Q] query tile
        set_roles();
        if (i == 0) chunk_scalars(Lc, M, g2, Mn, dec);
        // ---- inter term Q C for this wave's columns, both 32-row halves
        {
          float16_t hq[2];
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int r = 0; r < 16; ++r) hq[rb][r] = 0.0f;
          // Q fragments in batches of four k steps, the next batch's reads in
          // flight while the current batch is on the matrix cores
          constexpr int QB = 4;
          uint4 qa[2][QB][2];
          auto load_qa = [&](int sb, uint4 (&dst)[QB][2]) {
#pragma unroll
            for (int x = 0; x < QB; ++x)
#pragma unroll
              for (int rb = 0; rb < 2; ++rb)
                dst[x][rb] =
                    *reinterpret_cast<const uint4*>(s_q + (32 * rb + l32) * LDQ + 16 * (QB * sb + x) + 8 * h);
          };
          load_qa(0, qa[0]);
#pragma unroll
          for (int sb = 0; sb < NKS / QB; ++sb) {
            if (sb + 1 < NKS / QB) load_qa(sb + 1, qa[(sb + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int x = 0; x < QB; ++x) {
              const int s = QB * sb + x;
              const int q0 = 4 * (s & 1);
              const bf16x8_t bhi = as_bf16x8(
                  make_uint4(chi[s >> 1][q0], chi[s >> 1][q0 + 1], chi[s >> 1][q0 + 2], chi[s >> 1][q0 + 3]));
              const bf16x8_t blo = as_bf16x8(
                  make_uint4(clo[s >> 1][q0], clo[s >> 1][q0 + 1], clo[s >> 1][q0 + 2], clo[s >> 1][q0 + 3]));
#pragma unroll
              for (int rb = 0; rb < 2; ++rb) hq[rb] = mma32b(as_bf16x8(qa[sb & 1][x][rb]), bhi, hq[rb]);
#pragma unroll
              for (int rb = 0; rb < 2; ++rb) hq[rb] = mma32b(as_bf16x8(qa[sb & 1][x][rb]), blo, hq[rb]);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
          // to LDS as [column][row]: column 32 b + lane % 32, rows 32 rb + 8 q + 4 h .. + 3
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              *reinterpret_cast<float4*>(s_xt + (32 * wb + l32) * LDX + 32 * rb + 8 * q + 4 * h) =
                  make_float4(hq[rb][4 * q], hq[rb][4 * q + 1], hq[rb][4 * q + 2], hq[rb][4 * q + 3]);
        }
        // the last tile rebuilds float32 accumulators: decay times the old state
        float16_t cacc[last ? NKB : 1];
        if constexpr (last) {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              cacc[kb][2 * q] = dec * (__uint_as_float(chi[kb][q] << 16) + __uint_as_float(clo[kb][q] << 16));
              cacc[kb][2 * q + 1] =
                  dec * (__uint_as_float(chi[kb][q] & 0xffff0000u) + __uint_as_float(clo[kb][q] & 0xffff0000u));
            }
        }
        const int nkt = nkt_of(Lc, i);
        for (int j = 0; j < nkt; ++j) {
          if constexpr (last) {
            const int cur = ks & 1;
            const uint16_t* const s_k = s_kb[cur];
            const uint16_t* const s_v = s_vb[cur];
            const int key0 = j * TKV;
            // update C[., this wave's columns] += K^T (w . V) over 16-key
            // steps.  Transposing reads: lane j of each 16-lane group
            // addresses row 8 (grp / 2) + j / 4 and 4 rows further; the K
            // columns are taken in the state's permuted row order.
            const int grp = lane >> 4, jl = lane & 15;
            const int pc = 16 * (grp & 1) + 4 * (((jl & 1) << 1) | ((jl >> 1) & 1));
            const int kr0 = 8 * (grp >> 1) + (jl >> 2);
            int ktb[2][4];  // K rows kr0 and kr0 + 4, columns pc + 32 x
#pragma unroll
            for (int y = 0; y < 2; ++y)
#pragma unroll
              for (int x = 0; x < 4; ++x) ktb[y][x] = swz_base<DK>(kr0 + 4 * y, pc, x);
#pragma unroll
            for (int kk = 0; kk < TKV / 16; ++kk) {
              // w . V for keys 16 kk + 8 h + e as bf16 hi + lo
              const int vc = 32 * wb + 16 * (grp & 1) + 4 * (jl & 3);
              const uint2 v0r = lds_tr(s_v + swz<TVS>(16 * kk + kr0, vc));
              const uint2 v1r = lds_tr(s_v + swz<TVS>(16 * kk + kr0 + 4, vc));
              const float4 u0 = *reinterpret_cast<const float4*>(s_gu + key0 + 16 * kk + 8 * h);
              const float4 u1 = *reinterpret_cast<const float4*>(s_gu + key0 + 16 * kk + 8 * h + 4);
              // all K^T reads of the step go out before the arithmetic and the MFMAs
              uint4 akf[NKB];
#pragma unroll
              for (int kb = 0; kb < NKB; ++kb) {
                const int o = 128 * (kb >> 2) + 16 * kk * DK;
                const uint2 a0 = lds_tr(s_k + ktb[0][kb & 3] + o);
                const uint2 a1 = lds_tr(s_k + ktb[1][kb & 3] + o);
                akf[kb] = make_uint4(a0.x, a0.y, a1.x, a1.y);
              }
              __builtin_amdgcn_sched_barrier(0);
              const uint32_t vv[4] = {v0r.x, v0r.y, v1r.x, v1r.y};
              const float uu[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
              float ww[8];
#pragma unroll
              for (int e = 0; e < 8; ++e)
                ww[e] = __builtin_amdgcn_exp2f(SIG ? g2 + uu[e] : g2 + uu[e] - Mn);  // argument <= 0
              uint32_t hw[4], lw[4];
#pragma unroll
              for (int q = 0; q < 4; ++q)
                split_bf16x2(ww[2 * q] * __uint_as_float(vv[q] << 16),
                             ww[2 * q + 1] * __uint_as_float(vv[q] & 0xffff0000u), hw[q], lw[q]);
              const bf16x8_t bh_ = as_bf16x8(make_uint4(hw[0], hw[1], hw[2], hw[3]));
              const bf16x8_t bl_ = as_bf16x8(make_uint4(lw[0], lw[1], lw[2], lw[3]));
#pragma unroll
              for (int kb = 0; kb < NKB; ++kb) cacc[kb] = mma32b(as_bf16x8(akf[kb]), bh_, cacc[kb]);
#pragma unroll
              for (int kb = 0; kb < NKB; ++kb) cacc[kb] = mma32b(as_bf16x8(akf[kb]), bl_, cacc[kb]);
            }
          }
          ++ks;
          __syncthreads();  // [R] key tile
        }
        if constexpr (last) {
          if (c == Nc - 1 && p.C_out) write_state(cacc);
          split_state(cacc);
        }
      };
      for (int i = 0; i + 1 < nsub; ++i) sub_tile(std::false_type{}, i);
      sub_tile(std::true_type{}, nsub - 1);

      // ---- normaliser after the chunk: n = decay n + sum_t w_t k_t, the
      // sums over the chunk's keys formed by the intra role
      __syncthreads();  // [N] end of chunk
      if constexpr (!SIG) {
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) sum += s_np[w * DK + tb];
        nst = dec * nst + sum;
        put_n();
      }
      M = Mn;
    }

    // ---- final normaliser and stabiliser (the final C was written by the
    // last chunk's update, or copied from C0 for an empty sequence)
    if constexpr (!SIG) {
      if (slice == 0) {
        if (p.n_out) p.n_out[(size_t)bh * DK + tb] = nst;
        if (p.m_out && tb == 0) p.m_out[bh] = M * kLn2;
      }
    }
  }
}

template <int DK>
hipError_t launch_dk(const WalkParams& p, bool sig, hipStream_t stream) {
  const dim3 grid((unsigned)walk_workgroups(p.BH, p.DV));
  if (sig) hipLaunchKernelGGL((walk_kernel<DK, true>), grid, dim3(512), 0, stream, p);
  else hipLaunchKernelGGL((walk_kernel<DK, false>), grid, dim3(512), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

bool walk_supported(int DK, int DV, int L, bool bf16_inputs, bool split) {
  return bf16_inputs && split && DK == 256 && DV % kWalkSlice == 0 && L >= 64 && L <= kWalkMaxL;
}

long long walk_workgroups(int BH, int DV) { return (long long)BH * (DV / kWalkSlice); }

hipError_t launch_walk(const WalkParams& p, bool sig, hipStream_t stream) {
  if (p.DK == 256) return launch_dk<256>(p, sig, stream);
  return hipErrorInvalidValue;
}

}  // namespace mlstm
