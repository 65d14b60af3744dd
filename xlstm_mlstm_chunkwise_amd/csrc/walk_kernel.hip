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
// Wave w = (hf, cb), hf = w / 4, cb = w % 4, holds the state block
// C[128 hf .. 128 hf + 127][32 cb .. 32 cb + 31] (64 float32 values a lane)
// in matrix-core accumulators for the whole run.  Every chunk is processed in
// 64-row query tiles i; tile i takes the key tiles j <= i:
//   inter term   each wave forms Q_i[:, its DK half] . Cbar[its half, cb]
//                (Cbar = bf16 hi + lo split of its state block); the two DK
//                halves are summed through LDS, leaving wave (hf, cb) with
//                rows 32 hf .. 32 hf + 31, columns cb of H
//   scores       S^T = K_j . Q_i^T in 16 x 16 blocks: wave w takes queries
//                16 (w % 4) .. + 15 and keys 32 hf .. + 31
//   P = s S decay, shared through LDS as bf16 hi + lo planes
//   intra term   H += P . V_j for the wave's rows and columns
// and the last query tile of the chunk also does the state update
//   C = decay C + K_j^T (w . V_j)            (w . V_j as bf16 hi + lo,
//                                             formed from the V fragments)
// after its inter term has used the old state.  K and V tiles are double
// buffered: while the waves run P . V and the update on tile j, the next tile
// goes into the other buffers, so a key tile costs two barriers.  The four column slices of a
// head compute the same score tiles (that is the price of keeping C
// on-chip); they are placed on one XCD so their Q and K reads share an L2.
//
// State precision.  Between chunks a wave holds its state block as bf16
// hi + lo pairs (about 16 significant bits), the operand form of Q . Cbar;
// the last query tile of a chunk rebuilds float32 accumulators from them,
// applies the decay, accumulates the chunk's update on the matrix cores and
// splits the result again.  The rounding error this adds per chunk is
// relative 2^-17 of the state, and the decay keeps it from growing.
//
// Contraction order.  The state accumulators hold row m of each 32-row block
// at k index 32 kb + perm(m), where perm swaps the 4-row groups 1 and 2 of
// every 16 rows; the K^T operand of the update is read with that column
// permutation.  With it, the accumulator values a lane holds for a 16-deep k
// step of Q . Cbar are the k indices 8 (lane / 32) + e in natural order, so Q
// enters with plain 16-byte row reads.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace mlstm {
namespace {

constexpr int kWalkMaxL = 512;
constexpr int kWalkSlice = 128;

// K rows are stored unpadded with their 16-byte column groups XOR-swizzled by
// row, so that both the 16-byte row reads of the scores (16 consecutive rows,
// one group) and the transposing reads of the update (4 consecutive rows, 4
// consecutive groups) fall on distinct banks.
__device__ __forceinline__ int kswz(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }

// element offset of K tile element (row r, column c) for a row of DK elements
template <int DK>
__device__ __forceinline__ int koff(int r, int c) {
  return r * DK + (((c >> 3) ^ kswz(r)) << 3) + (c & 7);
}

// V tiles (kWalkSlice columns, unpadded): the 16-byte column groups of row r
// are XOR-ed with 4 (r % 4), which keeps both the 16-byte staging writes (one
// row, 16 groups) and the transposing reads (4 consecutive rows, 4
// consecutive groups) on distinct banks.
__device__ __forceinline__ int voff(int r, int c) {
  return r * kWalkSlice + (((c >> 3) ^ (4 * (r & 3))) << 3) + (c & 7);
}
// Fragment whose contraction axis runs down the rows of a swizzled V tile:
// lane l gets V[k0 + 8 (l / 32) + e][c0 + l % 32], e = 0..7.
__device__ __forceinline__ uint4 frag_tr_v(const uint16_t* X, int k0, int c0, int lane) {
  const int grp = lane >> 4, j = lane & 15;
  const int o = voff(k0 + 8 * (grp >> 1) + (j >> 2), c0 + 16 * (grp & 1) + 4 * (j & 3));
  const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)(X + o));
  const short4_t hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)(X + o + 4 * kWalkSlice));
  const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
  return make_uint4(a.x, a.y, b.x, b.y);
}

template <int DK, bool SIG>
__global__ __launch_bounds__(512) void walk_kernel(const WalkParams p) {
  constexpr int NT = 512, TQ = 64, TKV = 64, TVS = kWalkSlice;
  constexpr int LDQ = DK + 8;    // 16-byte row reads: 4 banks mod 64
  constexpr int LDP = TKV + 8;
  constexpr int DKH = DK / 2;    // DK rows of the state held by one wave
  constexpr int NKB = DKH / 32;  // its 32-row blocks
  constexpr int NKS = DKH / 16;  // 16-deep k steps over its half
  constexpr int NSS = DK / 32;   // 32-deep k steps of the scores
  constexpr int KG = DK / 8;     // 16-byte groups per Q / K row
  constexpr int QPT = TQ * KG / NT;
  constexpr int VG = TVS / 8;
  constexpr int VPT = TKV * VG / NT;
  static_assert(QPT * NT == TQ * KG && VPT * NT == TKV * VG, "staging split");
  static_assert(kWalkMaxL <= NT && DK <= NT, "one thread per position and per normaliser entry");
  static_assert(TKV * DK * 2 >= 8 * 16 * 64 * 4, "the inter-term exchange fits a K buffer");

  __shared__ __align__(16) uint16_t s_q[TQ * LDQ];
  __shared__ __align__(16) uint16_t s_kb[2][TKV * DK];   // K tiles, double buffered
  __shared__ __align__(16) uint16_t s_vb[2][TKV * TVS];  // V tiles, double buffered
  __shared__ __align__(16) uint16_t s_p[2 * TQ * LDP];  // P hi plane, then lo plane
  __shared__ __align__(16) float s_w[TKV];               // update weights of the current key tile
  __shared__ __align__(16) float s_gu[kWalkMaxL];
  __shared__ float s_gb[kWalkMaxL];
  __shared__ float s_gpm[SIG ? 1 : kWalkMaxL];
  __shared__ float s_row_r2[TQ], s_row_w[TQ], s_row_m2[TQ];
  __shared__ float s_den[3][TQ];  // inter part, intra parts of the two key halves
  __shared__ __align__(16) float s_inv[TQ];
  __shared__ __align__(16) float s_n[DK];
  uint16_t* const s_ph = s_p;
  uint16_t* const s_pl = s_p + TQ * LDP;
  float* const s_np = reinterpret_cast<float*>(s_p);  // n partial sums at the end of a chunk
  static_assert(2 * TQ * LDP * 2 >= 8 * DK * 4, "n partial sums fit the P planes");

  // Per-lane roles.  They are re-derived from a laundered thread index at the
  // top of every loop level, so the compiler rebuilds the LDS offsets that
  // depend on them instead of keeping them live across the walk.
  int tid, lane, wave, h, l32, l16, g4, hf, cb, qb;
  auto set_roles = [&]() {
    int t = (int)threadIdx.x;
    asm volatile("" : "+v"(t));
    int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    asm volatile("" : "+s"(w));
    tid = t;
    lane = t & 63;
    wave = w;
    h = lane >> 5;
    l32 = lane & 31;
    l16 = lane & 15;
    g4 = lane >> 4;
    hf = w >> 2;
    cb = w & 3;
    qb = w & 3;
  };
  set_roles();
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
  const uint16_t* Qh = static_cast<const uint16_t*>(p.Q) + (size_t)bh * S * DK;
  const uint16_t* Kh = static_cast<const uint16_t*>(p.K) + (size_t)bh * S * DK;
  const uint16_t* Vh = static_cast<const uint16_t*>(p.V) + (size_t)bh * S * DV + v0;
  const size_t gbase = (size_t)bh * S;
  auto vcol = [&]() { return v0 + 32 * cb + l32; };  // the state / H column of this lane

  // ---- state.  Accumulator register r of block kb holds C[dk][vcol] with
  // dk = DKH hf + 32 kb + perm(row of r); chi / clo hold the block as bf16
  // hi + lo words, word q packing registers 2q (low half) and 2q + 1.
  auto state_row = [&](int kb, int r) {
    const int j = r >> 2;
    return DKH * hf + 32 * kb + 16 * (j >> 1) + 8 * h + 4 * (j & 1) + (r & 3);
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
        make_rsrc(p.C0 ? p.C0 + (size_t)bh * DK * DV : p.gb2, p.C0 ? (uint32_t)(DK * DV * 4) : 0u);
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
  if (!SIG && tid < DK) s_n[tid] = p.n0 ? p.n0[(size_t)bh * DK + tid] : 0.0f;
  float M = (!SIG && p.m0) ? p.m0[bh] * kLog2e : 0.0f;  // stabiliser, log2 units

  // ---- global loads, one step ahead.  Q tiles in (chunk, query tile)
  // order; K / V tiles in (chunk, query tile, key tile <= query tile) order.
  auto nsub_of = [&](int c) { return (min(L, S - c * L) + TQ - 1) / TQ; };
  uint4 qpre[QPT], kpre[QPT], vpre[VPT];
  float gpre_u, gpre_b, gpre_pm;
  int qc = 0, qi = 0;          // next Q tile to load
  int kc = 0, ki = 0, kj = 0;  // next K / V tile to load
  auto load_q = [&]() {
    if (qc >= Nc) return;
    const int t0 = qc * L, Lc = min(L, S - t0), r0 = qi * TQ;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(Qh + (size_t)(t0 + r0) * DK, (uint32_t)((Lc - r0) * DK * 2));
#pragma unroll
    for (int i = 0; i < QPT; ++i) qpre[i] = buf_load16(rq, tid * 16, i * NT * 16);
    if (++qi >= nsub_of(qc)) {
      qi = 0;
      ++qc;
    }
  };
  auto load_kv = [&]() {
    if (kc >= Nc) return;
    const int t0 = kc * L, Lc = min(L, S - t0), k0 = kj * TKV;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kh + (size_t)(t0 + k0) * DK, (uint32_t)((Lc - k0) * DK * 2));
    const __amdgpu_buffer_rsrc_t rv =
        make_rsrc(Vh + (size_t)(t0 + k0) * DV, (uint32_t)(((Lc - k0 - 1) * DV + TVS) * 2));
#pragma unroll
    for (int i = 0; i < QPT; ++i) kpre[i] = buf_load16(rk, tid * 16, i * NT * 16);
#pragma unroll
    for (int i = 0; i < VPT; ++i)
      vpre[i] = buf_load16(rv, ((tid / VG) * DV + (tid % VG) * 8) * 2, i * (NT / VG) * DV * 2);
    if (++kj > ki) {
      kj = 0;
      if (++ki >= nsub_of(kc)) {
        ki = 0;
        ++kc;
      }
    }
  };
  auto load_gates = [&](int c) {
    if (c >= Nc) return;
    const int t0 = c * L, Lc = min(L, S - t0);
    const bool ok = tid < Lc;
    gpre_u = ok ? p.gu2[gbase + t0 + tid] : 0.0f;
    gpre_b = ok ? p.gb2[gbase + t0 + tid] : 0.0f;
    gpre_pm = (!SIG && ok) ? p.gpm2[gbase + t0 + tid] : 0.0f;
  };
  // K / V tile n of the (chunk, query tile, key tile) sequence sits in
  // buffer n % 2; ks counts the tiles consumed.  stage() writes the tile held
  // in registers into the buffer after the current one and requests the
  // next; have_kv says whether registers hold a tile.
  bool have_kv = false;
  int ks = 0;
  // piece e of this thread is K row tid / KG + e NT / KG, column group
  // tid % KG (the swizzle of a row repeats every 16 rows), and V row
  // tid / VG + e NT / VG, column group tid % VG (period 4)
  static_assert((NT / KG) % 16 == 0 && (NT / VG) % 4 == 0, "swizzle period");
  auto stage = [&](int buf) {
    if (have_kv) {
      const int kst = koff<DK>(tid / KG, (tid % KG) * 8);
#pragma unroll
      for (int e = 0; e < QPT; ++e) *reinterpret_cast<uint4*>(s_kb[buf] + kst + e * (NT / KG) * DK) = kpre[e];
      const int vst = voff(tid / VG, (tid % VG) * 8);
#pragma unroll
      for (int e = 0; e < VPT; ++e) *reinterpret_cast<uint4*>(s_vb[buf] + vst + e * (NT / VG) * TVS) = vpre[e];
    }
    have_kv = kc < Nc;
    load_kv();
  };
  load_gates(0);
  load_q();
  have_kv = kc < Nc;
  load_kv();
  stage(0);

  float np[8];  // n partial sums of this thread's key columns (exp gate)

  for (int c = 0; c < Nc; ++c) {
    set_roles();
    const int t0 = c * L, Lc = min(L, S - t0);
    const int nsub = (Lc + TQ - 1) / TQ;
    // u past the end of a short last chunk is -inf: those keys (zero rows)
    // get weight exactly zero
    if (tid < L) {
      s_gu[tid] = tid < Lc ? gpre_u : -INFINITY;
      s_gb[tid] = gpre_b;
      if constexpr (!SIG) s_gpm[tid] = gpre_pm;
    }
    load_gates(c + 1);
#pragma unroll
    for (int e = 0; e < 8; ++e) np[e] = 0.0f;
    __syncthreads();
    // chunk scalars: stabiliser after the chunk, decay of the old state
    const float g2 = s_gb[Lc - 1];
    float Mn = 0.0f, dec;
    if constexpr (SIG) {
      dec = exp2f(g2);
    } else {
      Mn = g2 + fmaxf(M, s_gpm[Lc - 1]);
      dec = exp2f(g2 + M - Mn);
    }
    // weight of step sigma in the state update (0 past the chunk end)
    auto upd_w = [&](int sigma) -> float {
      return SIG ? exp2f(g2 + s_gu[sigma]) : exp2f(g2 + s_gu[sigma] - Mn);
    };

    // query tile i; LAST: the chunk's last tile, which also updates the state
    auto sub_tile = [&](auto last_c, int i) {
      constexpr bool last = decltype(last_c)::value;
      set_roles();
      const int row0 = i * TQ;
      // per-row terms: exponent offset r2 of P (with log2 s; -inf past the
      // chunk end), weight of the inter term, stabiliser m (log2 units)
      if (tid < TQ) {
        const int tau = row0 + tid;
        float r2 = -INFINITY, wr = 0.0f, m2 = 0.0f;
        if (tau < Lc) {
          const float b2 = s_gb[tau];
          if constexpr (SIG) {
            r2 = b2 + log2_scale;
            wr = exp2f(b2);
          } else {
            const float mx = fmaxf(M, s_gpm[tau]);
            r2 = log2_scale - mx;
            wr = exp2f(M - mx);
            m2 = b2 + mx;
          }
        }
        s_row_r2[tid] = r2;
        s_row_w[tid] = wr * scale;
        s_row_m2[tid] = m2;
      }
#pragma unroll
      for (int e = 0; e < QPT; ++e) {
        const int idx = tid + e * NT;
        *reinterpret_cast<uint4*>(s_q + (idx / KG) * LDQ + (idx % KG) * 8) = qpre[e];
      }
      load_q();
      __syncthreads();

      // this wave's 16 queries as B fragments of the 16 x 16 x 32 score blocks
      // (the Q tile stays in LDS until the next query tile)
      auto qs = [&](int s) { return *reinterpret_cast<const uint4*>(s_q + (16 * qb + l16) * LDQ + 32 * s + 8 * g4); };

      // ---- inter term over this wave's DK half, both 32-row halves of the tile
      float16_t part[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int r = 0; r < 16; ++r) part[rb][r] = 0.0f;
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        uint4 a[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          a[rb] = *reinterpret_cast<const uint4*>(s_q + (32 * rb + l32) * LDQ + DKH * hf + 16 * s + 8 * h);
        const int q0 = 4 * (s & 1);
        const bf16x8_t bhi =
            as_bf16x8(make_uint4(chi[s >> 1][q0], chi[s >> 1][q0 + 1], chi[s >> 1][q0 + 2], chi[s >> 1][q0 + 3]));
        const bf16x8_t blo =
            as_bf16x8(make_uint4(clo[s >> 1][q0], clo[s >> 1][q0 + 1], clo[s >> 1][q0 + 2], clo[s >> 1][q0 + 3]));
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          part[rb] = mma32b(as_bf16x8(a[rb]), bhi, part[rb]);
          part[rb] = mma32b(as_bf16x8(a[rb]), blo, part[rb]);
        }
      }
      // normaliser contribution of the state, s e^{M - m} q . n: thread t
      // takes row t / 8 over DK / 8 of the entries
      if constexpr (!SIG) {
        const int row = tid >> 3, seg = (tid & 7) * (DK / 8);
        float d = 0.0f;
#pragma unroll
        for (int g = 0; g < DK / 64; ++g) {
          const uint4 qv = *reinterpret_cast<const uint4*>(s_q + row * LDQ + seg + 8 * g);
          const float4 n0 = *reinterpret_cast<const float4*>(s_n + seg + 8 * g);
          const float4 n1 = *reinterpret_cast<const float4*>(s_n + seg + 8 * g + 4);
          d += __uint_as_float(qv.x << 16) * n0.x + __uint_as_float(qv.x & 0xffff0000u) * n0.y;
          d += __uint_as_float(qv.y << 16) * n0.z + __uint_as_float(qv.y & 0xffff0000u) * n0.w;
          d += __uint_as_float(qv.z << 16) * n1.x + __uint_as_float(qv.z & 0xffff0000u) * n1.y;
          d += __uint_as_float(qv.w << 16) * n1.z + __uint_as_float(qv.w & 0xffff0000u) * n1.w;
        }
        d += __shfl_xor(d, 1, 64);
        d += __shfl_xor(d, 2, 64);
        d += __shfl_xor(d, 4, 64);
        if ((tid & 7) == 0) s_den[0][row] = d * s_row_w[row];
      }
      // the other half's rows go to the partner wave (same columns, other DK
      // half), through the K buffer that does not hold the next tile
      float* const s_x = reinterpret_cast<float*>(s_kb[(ks & 1) ^ 1]);
#pragma unroll
      for (int r = 0; r < 16; ++r) s_x[(wave * 16 + r) * 64 + lane] = part[1 - hf][r];
      __syncthreads();
      float16_t hacc = part[hf];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        hacc[r] += s_x[((wave ^ 4) * 16 + r) * 64 + lane];
        hacc[r] *= s_row_w[32 * hf + 8 * (r >> 2) + 4 * h + (r & 3)];
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
      float dpart = 0.0f;
      const int tl = 16 * qb + l16;  // query of this lane in the score block, within the tile
      const float r2 = s_row_r2[tl];

      // ---- key tiles: tile j is in buffers ks % 2 (staged one tile ahead)
      for (int j = 0; j <= i; ++j) {
        const int key0 = j * TKV;
        const int cur = ks & 1;
        const uint16_t* const s_k = s_kb[cur];
        const uint16_t* const s_v = s_vb[cur];
        if constexpr (last) {
          if (tid < TKV) s_w[tid] = upd_w(key0 + tid);
        }

        // scores: keys 32 hf + 16 kb + [0, 16) x this wave's 16 queries, then
        // P = S 2^{r2 + u} (rows past the chunk end have r2 = -inf and keys
        // past it u = -inf, so only the diagonal tile needs the causal
        // select).  NLIVE key blocks hold keys at or below some query of the
        // wave; the others are above the diagonal and written as zero, since
        // P . V reads 32-row pieces.
        auto scores = [&](auto nlive_c, auto diag_c) {
          constexpr int NLIVE = decltype(nlive_c)::value;
          constexpr bool diag = decltype(diag_c)::value;
          float4_t sacc[2];
#pragma unroll
          for (int kb = 0; kb < NLIVE; ++kb) sacc[kb] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int s = 0; s < NSS; ++s) {
            const uint4 b = qs(s);
#pragma unroll
            for (int kb = 0; kb < NLIVE; ++kb) {
              const uint4 a = *reinterpret_cast<const uint4*>(s_k + koff<DK>(32 * hf + 16 * kb + l16, 32 * s + 8 * g4));
              sacc[kb] = mma16b(as_bf16x8(a), as_bf16x8(b), sacc[kb]);
            }
          }
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            const int kl = 32 * hf + 16 * kb + 4 * g4;  // first of this lane's 4 keys, within the tile
            if (kb >= NLIVE) {
              *reinterpret_cast<uint2*>(s_ph + tl * LDP + kl) = make_uint2(0u, 0u);
              *reinterpret_cast<uint2*>(s_pl + tl * LDP + kl) = make_uint2(0u, 0u);
              continue;
            }
            const float4 u4 = *reinterpret_cast<const float4*>(s_gu + key0 + kl);
            const float uu[4] = {u4.x, u4.y, u4.z, u4.w};
            float val[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              val[e] = sacc[kb][e] * __builtin_amdgcn_exp2f(r2 + uu[e]);
              if constexpr (diag) val[e] = (kl + e <= tl) ? val[e] : 0.0f;
              dpart += val[e];
            }
            uint2 ph, pl;
            split_bf16x2(val[0], val[1], ph.x, pl.x);
            split_bf16x2(val[2], val[3], ph.y, pl.y);
            *reinterpret_cast<uint2*>(s_ph + tl * LDP + kl) = ph;
            *reinterpret_cast<uint2*>(s_pl + tl * LDP + kl) = pl;
          }
        };
        if (j < i) {
          scores(std::integral_constant<int, 2>{}, std::false_type{});
        } else if (32 * hf + 16 <= 16 * qb + 15) {
          scores(std::integral_constant<int, 2>{}, std::true_type{});
        } else if (32 * hf <= 16 * qb + 15) {
          scores(std::integral_constant<int, 1>{}, std::true_type{});
        } else {
          scores(std::integral_constant<int, 0>{}, std::true_type{});
        }
        __syncthreads();

        // intra term H += P . V over 16-key steps (rows 32 hf.., columns cb)
        // and, on the last query tile, the state update C[this wave's DK
        // half, cb] += K^T (w . V) from the same V fragments
        [[maybe_unused]] int kbase[NKB][2];
        if constexpr (last) {
          const int grp = lane >> 4, jl = lane & 15;
          const int pc = 16 * (grp & 1) + 4 * (((jl & 1) << 1) | ((jl >> 1) & 1));  // permuted column group
          // rows kr0 + 16 kk and kr0 + 4 + 16 kk: the swizzle repeats every 16
          // rows, so each column block needs two base offsets
          const int kr0 = 8 * (grp >> 1) + (jl >> 2);
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
            kbase[kb][0] = koff<DK>(kr0, DKH * hf + 32 * kb + pc);
            kbase[kb][1] = koff<DK>(kr0 + 4, DKH * hf + 32 * kb + pc);
          }
        }
#pragma unroll
        for (int kk = 0; kk < TKV / 16; ++kk) {
          const bool pv_live = !(j == i && 16 * kk > 32 * hf + 31);  // above the diagonal: P is zero
          if (!last && !pv_live) continue;
          const uint4 vraw = frag_tr_v(s_v, 16 * kk, 32 * cb, lane);
          if (pv_live) {
            const uint4 ahi = frag_row_u(s_ph, LDP, 32 * hf, 16 * kk, lane);
            const uint4 alo = frag_row_u(s_pl, LDP, 32 * hf, 16 * kk, lane);
            hacc = mma32b(as_bf16x8(ahi), as_bf16x8(vraw), hacc);
            hacc = mma32b(as_bf16x8(alo), as_bf16x8(vraw), hacc);
          }
          if constexpr (last) {
            // w . V for keys 16 kk + 8 (lane / 32) + e as bf16 hi + lo
            const float4 w0 = *reinterpret_cast<const float4*>(s_w + 16 * kk + 8 * h);
            const float4 w1 = *reinterpret_cast<const float4*>(s_w + 16 * kk + 8 * h + 4);
            const uint32_t vv[4] = {vraw.x, vraw.y, vraw.z, vraw.w};
            const float ww[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
            uint32_t hw[4], lw[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
              split_bf16x2(ww[2 * q] * __uint_as_float(vv[q] << 16), ww[2 * q + 1] * __uint_as_float(vv[q] & 0xffff0000u),
                           hw[q], lw[q]);
            const bf16x8_t bh_ = as_bf16x8(make_uint4(hw[0], hw[1], hw[2], hw[3]));
            const bf16x8_t bl_ = as_bf16x8(make_uint4(lw[0], lw[1], lw[2], lw[3]));
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
              const short4_t x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (__attribute__((address_space(3))) short4_t*)(s_k + kbase[kb][0] + 16 * kk * DK));
              const short4_t x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (__attribute__((address_space(3))) short4_t*)(s_k + kbase[kb][1] + 16 * kk * DK));
              const uint2 a0 = __builtin_bit_cast(uint2, x0), a1 = __builtin_bit_cast(uint2, x1);
              const bf16x8_t ak = as_bf16x8(make_uint4(a0.x, a0.y, a1.x, a1.y));
              cacc[kb] = mma32b(ak, bh_, cacc[kb]);
              cacc[kb] = mma32b(ak, bl_, cacc[kb]);
            }
          }
        }
        // n partial sums (exp gate, last query tile): this thread's K pieces
        // of the tile, weighted
        if constexpr (!SIG && last) {
          const int kst = koff<DK>(tid / KG, (tid % KG) * 8);
#pragma unroll
          for (int e = 0; e < QPT; ++e) {
            const float w = s_w[tid / KG + e * (NT / KG)];
            const uint4 kv = *reinterpret_cast<const uint4*>(s_k + kst + e * (NT / KG) * DK);
            const uint32_t kw[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              np[2 * q] += w * __uint_as_float(kw[q] << 16);
              np[2 * q + 1] += w * __uint_as_float(kw[q] & 0xffff0000u);
            }
          }
        }
        // the next tile into the other buffers (last read before the previous
        // barrier)
        stage(cur ^ 1);
        ++ks;
        __syncthreads();
      }
      if constexpr (last) {
        if (c == Nc - 1 && p.C_out) write_state(cacc);
        split_state(cacc);
      }

      // ---- normaliser and H for this query tile
      set_roles();
      if constexpr (!SIG) {
        dpart += __shfl_xor(dpart, 16, 64);
        dpart += __shfl_xor(dpart, 32, 64);
        if (lane < 16) s_den[1 + hf][16 * qb + lane] = dpart;
        __syncthreads();
        if (tid < TQ) {
          const float d = s_den[0][tid] + s_den[1][tid] + s_den[2][tid];
          s_inv[tid] = 1.0f / (fmaxf(fabsf(d), exp2f(-s_row_m2[tid])) + p.eps);
        }
        __syncthreads();
      }
      auto store_h = [&](auto esize) {
        constexpr int E = decltype(esize)::value;
        const __amdgpu_buffer_rsrc_t rh =
            make_rsrc(static_cast<const char*>(p.H) + ((gbase + t0 + row0) * DV + v0) * E,
                      (uint32_t)(((Lc - row0 - 1) * DV + TVS) * E));
        const int hvoff = ((32 * hf + 4 * h) * DV + 32 * cb + l32) * E;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          float4 inv = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
          if constexpr (!SIG) inv = *reinterpret_cast<const float4*>(s_inv + 32 * hf + 8 * r4 + 4 * h);
          const float iv[4] = {inv.x, inv.y, inv.z, inv.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float hv = hacc[4 * r4 + q] * iv[q];
            const int soff = (8 * r4 + q) * DV * E;
            // non-temporal (aux 2): H is written once and never read here
            if constexpr (E == 2)
              __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(hv), rh, hvoff, soff, 2);
            else
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(hv), rh, hvoff, soff, 2);
          }
        }
      };
      if (p.h_bf16) store_h(std::integral_constant<int, 2>{});
      else store_h(std::integral_constant<int, 4>{});
    };
    for (int i = 0; i + 1 < nsub; ++i) sub_tile(std::false_type{}, i);
    sub_tile(std::true_type{}, nsub - 1);

    // ---- normaliser after the chunk: n = decay n + sum_t w_t k_t
    if constexpr (!SIG) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int o = KG; o < 64; o <<= 1) np[e] += __shfl_xor(np[e], o, 64);
      if (lane < KG) {
#pragma unroll
        for (int e = 0; e < 8; ++e) s_np[wave * DK + lane * 8 + e] = np[e];
      }
      __syncthreads();
      if (tid < DK) {
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < 8; ++w) sum += s_np[w * DK + tid];
        s_n[tid] = dec * s_n[tid] + sum;
      }
      M = Mn;
      __syncthreads();
    }
  }

  // ---- final normaliser and stabiliser (the final C was written by the last
  // chunk's update, or copied from C0 for an empty sequence)
  set_roles();
  if constexpr (!SIG) {
    if (slice == 0) {
      if (p.n_out && tid < DK) p.n_out[(size_t)bh * DK + tid] = s_n[tid];
      if (p.m_out && tid == 0) p.m_out[bh] = M * kLn2;
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
