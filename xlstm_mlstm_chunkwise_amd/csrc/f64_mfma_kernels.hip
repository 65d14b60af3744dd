// Float64 evaluation of both stages of the chunkwise mLSTM forward pass on the
// fp64 matrix cores (precision mode MLSTM_PREC_F64; gfx950
// v_mfma_f64_16x16x4_f64).
//
// Same arithmetic as the vector-unit fp64 kernel (f64_kernels.hip): the
// chunkwise form (TFLA abstract: an inter-chunk recurrence plus a parallel
// intra-chunk part; the mLSTM cell with its normaliser and max-state, "xLSTM:
// the NX-AI repository behind the extended LSTM architecture", section
// "Exponential gating, matrix memory, and why the kernels decide
// everything"), every value and every sum in fp64.  The fp64 matrix cores
// have the same peak as the fp64 vector units on this chip, but each 16 x 16
// x 4 product takes its two operands as one double per lane, so a product
// needs two LDS values per 32 FLOP of a lane where a 4 x 4 register block on
// the vector units needs eight.
//
// Operand layout of v_mfma_f64_16x16x4_f64: lane l supplies A[l % 16][l / 16]
// and B[l / 16][l % 16]; register r of the accumulator holds
// D[4 r + l / 16][l % 16] (rows interleaved over the four lane groups, unlike
// the float32 16 x 16 products, whose register r holds row 4 (l / 16) + r).
// Which contraction index a slot stands for is free as long as A and B agree:
// for the four products of a 16-deep step, slot g = l / 16 of product s
// stands for index 4 g + s, so a lane reads its four operands of a step as
// four consecutive elements.  The score accumulator of a 16-key block is S^T
// (keys as rows), whose register r in lane l is the score of query l % 16
// with key 4 r + l / 16: exactly the A operand of product r of the P.V step
// when slot g of product r stands for key 4 r + g.  The staged value tile
// stores the keys of each 16-key block in that order (key 4 r + g at position
// 4 g + r), so a lane again reads four consecutive elements and P never
// leaves the registers.
#include <type_traits>

#include "device_common.h"
#include "f64_common.h"
#include "kernels.h"
#include "tile_order.h"

namespace mlstm {
namespace {

using namespace f64;

typedef double double4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ double4_t mma_f64(double a, double b, double4_t c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

// Four consecutive staged inputs (8 bytes of bf16 or 16 bytes of float32),
// widened to double.
template <typename TIn>
__device__ __forceinline__ void lds4(const TIn* p, double (&x)[4]);
template <>
__device__ __forceinline__ void lds4<bf16_t>(const bf16_t* p, double (&x)[4]) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  x[0] = (double)__uint_as_float(u.x << 16);
  x[1] = (double)__uint_as_float(u.x & 0xffff0000u);
  x[2] = (double)__uint_as_float(u.y << 16);
  x[3] = (double)__uint_as_float(u.y & 0xffff0000u);
}
template <>
__device__ __forceinline__ void lds4<float>(const float* p, double (&x)[4]) {
  const float4 u = *reinterpret_cast<const float4*>(p);
  x[0] = u.x;
  x[1] = u.y;
  x[2] = u.z;
  x[3] = u.w;
}

// 16 bytes of inputs per global load: 8 bf16 or 4 float32.
template <typename TIn>
struct Vec16 {
  static constexpr int N = 16 / sizeof(TIn);
};

// ---------------------------------------------------------------------------
// Stage one: a 64 x TVC tile of C per workgroup (TVC = 64 or 32), walking the
// chunks of its head.  Wave w owns state rows 16 w .. 16 w + 15 of the tile
// and its TVC / 16 column blocks (accumulator register r of block cb: row
// 16 w + 4 r + l / 16, column 16 cb + l % 16).  Per chunk the gated keys (K w, fp64) and the values
// are staged transposed, 32 steps at a time, and C += (K w)^T V runs on the
// matrix cores.

constexpr int kSTB = 32;          // time steps per staging block
constexpr int kSLD = kSTB + 4;    // row stride (doubles) of the transposed tiles

// One thread's share of a staging block, held in registers from its loads to
// its LDS stores: step tid % 32 of the block, columns 8 (tid / 32) .. + 7 of
// the 64-wide K and V slices (one 16-byte load each for bf16, two for
// float32).
template <typename TIn>
struct StageRegs {
  static constexpr int NV = 8 * (int)sizeof(TIn) / 16;
  uint4 k[NV], v[NV];
};

template <typename TIn>
__device__ __forceinline__ void widen8(const uint4 (&u)[StageRegs<TIn>::NV], double (&x)[8]);
template <>
__device__ __forceinline__ void widen8<bf16_t>(const uint4 (&u)[1], double (&x)[8]) {
  const uint32_t w[4] = {u[0].x, u[0].y, u[0].z, u[0].w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = (double)__uint_as_float(w[i] << 16);
    x[2 * i + 1] = (double)__uint_as_float(w[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void widen8<float>(const uint4 (&u)[2], double (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    x[4 * i] = (double)__uint_as_float(u[i].x);
    x[4 * i + 1] = (double)__uint_as_float(u[i].y);
    x[4 * i + 2] = (double)__uint_as_float(u[i].z);
    x[4 * i + 3] = (double)__uint_as_float(u[i].w);
  }
}

// TVC: columns of the C tile (64, or 32 to give heads with few tiles twice
// the workgroups: two per CU instead of one).
template <typename TIn, bool SIG, int TVC>
__global__ __launch_bounds__(256) void states_f64m_kernel(const StatesParams p) {
  constexpr int NCB = TVC / 16;  // 16-column blocks of a wave
  __shared__ double s_w[kMaxL];
  __shared__ double s_tot[4];  // wave totals of the block scans
  __shared__ double s_g;
  __shared__ __align__(32) double s_kwt[64 * kSLD];  // [state row][step]
  __shared__ __align__(32) double s_vt[64 * kSLD];   // [column][step]

  const int bh = blockIdx.x, kt = blockIdx.y, vt = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, l16 = lane & 15;
  const int S = p.S, DK = p.DK, DV = p.DV, L = p.L, Nc = p.Nc;
  const TIn* K = static_cast<const TIn*>(p.K) + (size_t)bh * S * DK;
  const TIn* V = static_cast<const TIn*>(p.V) + (size_t)bh * S * DV;
  const float* ig = p.i_pre + (size_t)bh * S;
  const float* fg = p.f_pre + (size_t)bh * S;
  const bool own_n = !SIG && vt == 0;
  double* Cs = reinterpret_cast<double*>(p.C_states);
  double* ns = reinterpret_cast<double*>(p.n_states);
  double* ms = reinterpret_cast<double*>(p.m_states);
  auto krow = [&](int r) { return kt * 64 + 16 * w + 4 * r + g; };
  auto vcol = [&](int cb) { return vt * TVC + 16 * cb + l16; };

  const int st_t = tid & 31, st_c = 8 * (tid >> 5);  // this thread's staging step and columns
  const bool st_v = st_c < TVC;  // this thread also stages values
  StageRegs<TIn> cur;
  auto load_block = [&](int t0, int Lc, int tb, StageRegs<TIn>& sr) {
    // steps past the chunk read row t0 (in bounds) and are zeroed after
    const bool ok = tb + st_t < Lc;
    const size_t row = (size_t)t0 + (ok ? tb + st_t : 0);
    const uint4* kp = reinterpret_cast<const uint4*>(K + row * DK + kt * 64 + st_c);
    const uint4* vp = reinterpret_cast<const uint4*>(V + row * DV + vt * TVC + (st_v ? st_c : 0));
    const uint32_t keep = ok ? 0xffffffffu : 0u;
#pragma unroll
    for (int i = 0; i < StageRegs<TIn>::NV; ++i) {
      const uint4 a = kp[i];
      sr.k[i] = make_uint4(a.x & keep, a.y & keep, a.z & keep, a.w & keep);
      if (st_v) {
        const uint4 b = vp[i];
        sr.v[i] = make_uint4(b.x & keep, b.y & keep, b.z & keep, b.w & keep);
      }
    }
  };

  double4_t acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      acc[cb][r] = p.C0 ? (double)p.C0[(size_t)bh * DK * DV + (size_t)krow(r) * DV + vcol(cb)] : 0.0;
  double nreg = 0.0;  // n for state row kt * 64 + tid (tid < 64)
  if (own_n && tid < 64 && p.n0) nreg = p.n0[(size_t)bh * DK + kt * 64 + tid];
  double M = (!SIG && p.m0) ? (double)p.m0[bh] : 0.0;

  for (int c = 0; c <= Nc; ++c) {
    // the state entering chunk c (c == Nc: the final state)
    double* Cst = Cs + ((size_t)bh * (Nc + 1) + c) * DK * DV;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) Cst[(size_t)krow(r) * DV + vcol(cb)] = acc[cb][r];
    if (own_n && tid < 64) ns[((size_t)bh * (Nc + 1) + c) * DK + kt * 64 + tid] = nreg;
    if (!SIG && kt == 0 && vt == 0 && tid == 0) ms[(size_t)bh * (Nc + 1) + c] = M;
    if (c == Nc) break;

    // gates of the chunk: b = inclusive sum of log sigmoid(f), the key
    // weights and the decay of the old state (stabilised for the exp gate);
    // the chunk's first staging block is loaded meanwhile
    const int t0 = c * L, Lc = min(L, S - t0);
    load_block(t0, Lc, 0, cur);
    double b[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int pos = 4 * tid + e;
      b[e] = pos < Lc ? log_sigmoid_d((double)fg[t0 + pos]) : 0.0;
    }
    block_scan4_d<false>(b, s_tot);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (4 * tid + e == Lc - 1) s_g = b[e];
    __syncthreads();
    const double gsum = s_g;
    double a[4], amax = -INFINITY;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int pos = 4 * tid + e;
      if (pos < Lc) {
        const double it = (double)ig[t0 + pos];
        a[e] = gsum - b[e] + (SIG ? log_sigmoid_d(it) : it);
        amax = fmax(amax, a[e]);
      } else {
        a[e] = -INFINITY;
      }
    }
    double decay;
    if constexpr (SIG) {
      decay = exp(gsum);
#pragma unroll
      for (int e = 0; e < 4; ++e) s_w[4 * tid + e] = (4 * tid + e < Lc) ? exp(a[e]) : 0.0;
    } else {
      amax = block_max_d(amax, s_tot);
      const double Mn = fmax(gsum + M, amax);
      decay = exp(gsum + M - Mn);
#pragma unroll
      for (int e = 0; e < 4; ++e) s_w[4 * tid + e] = (4 * tid + e < Lc) ? exp(a[e] - Mn) : 0.0;
      M = Mn;
    }
    __syncthreads();
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[cb] *= decay;
    nreg *= decay;

    for (int tb = 0; tb < Lc; tb += kSTB) {
      // 32 steps x 64 state rows of K w and 32 steps x 64 columns of V,
      // transposed (steps past the chunk hold zeros); the next block's loads
      // go out before this block's products
      {
        double kx[8], vx[8];
        widen8<TIn>(cur.k, kx);
        widen8<TIn>(cur.v, vx);
        const double wt = s_w[tb + st_t];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          s_kwt[(st_c + e) * kSLD + st_t] = kx[e] * wt;
          if (st_v) s_vt[(st_c + e) * kSLD + st_t] = vx[e];
        }
      }
      if (tb + kSTB < Lc) load_block(t0, Lc, tb + kSTB, cur);
      __syncthreads();
      if (own_n && tid < 64) {
        double sacc = 0.0;
        for (int t = 0; t < kSTB; ++t) sacc += s_kwt[tid * kSLD + t];
        nreg += sacc;
      }
#pragma unroll
      for (int s0 = 0; s0 < kSTB; s0 += 16) {
        const double4_t ka = *reinterpret_cast<const double4_t*>(s_kwt + (16 * w + l16) * kSLD + s0 + 4 * g);
        double4_t vb[NCB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
          vb[cb] = *reinterpret_cast<const double4_t*>(s_vt + (16 * cb + l16) * kSLD + s0 + 4 * g);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) acc[cb] = mma_f64(ka[s], vb[cb][s], acc[cb]);
      }
      __syncthreads();
    }
  }
  if (p.C_out)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        p.C_out[(size_t)bh * DK * DV + (size_t)krow(r) * DV + vcol(cb)] = (float)acc[cb][r];
  if (own_n && p.n_out && tid < 64) p.n_out[(size_t)bh * DK + kt * 64 + tid] = (float)nreg;
  if (!SIG && p.m_out && kt == 0 && vt == 0 && tid == 0) p.m_out[bh] = (float)M;
}

// ---------------------------------------------------------------------------
// Stage two: 64 rows x TV columns of H per workgroup.  Wave w owns rows
// 16 w .. 16 w + 15 of the tile and its TV / 16 column blocks (accumulator
// register r of block cb: row 16 w + 4 r + l / 16, column 16 cb + l % 16).
// Q and K tiles are staged as inputs, row-major; V transposed ([column][key],
// keys permuted within 16-key blocks) and the chunk state in 16-row blocks
// transposed ([column][row]).

template <typename TIn, int DK, int TV>
struct F64mLayout {
  static constexpr int LDI = DK + 16 / (int)sizeof(TIn);   // 16-byte aligned rows of Q and K
  static constexpr int LDV = 64 + 16 / (int)sizeof(TIn);   // transposed V: 64 keys per column
  static constexpr int LDC = 16 + 4;                        // transposed state block, 32-byte rows
  static constexpr int K_BYTES = 64 * LDI * (int)sizeof(TIn);
  static constexpr int C_BYTES = TV * LDC * 8;
  static constexpr int V_BYTES = TV * LDV * (int)sizeof(TIn);
  // One region holds, phase by phase, the gate sums b (kMaxL doubles), the
  // state blocks of the inter-chunk term and the key tiles; the scan scratch
  // (4 doubles) of the gate phase lives in the value tile's space.
  static constexpr int A_BYTES = K_BYTES > C_BYTES ? (K_BYTES > kMaxL * 8 ? K_BYTES : kMaxL * 8)
                                                   : (C_BYTES > kMaxL * 8 ? C_BYTES : kMaxL * 8);
  static_assert(V_BYTES >= 4 * 8, "scan scratch must fit in the value tile");
};

template <typename TIn, bool SIG, int DK, int TV>
__global__ __launch_bounds__(256) void hintra_f64m_kernel(const HintraParams p) {
  typedef F64mLayout<TIn, DK, TV> Ly;
  constexpr int NCB = TV / 16;
  constexpr int VN = Vec16<TIn>::N;
  __shared__ __align__(32) TIn s_q[64 * Ly::LDI];
  __shared__ __align__(32) unsigned char s_araw[Ly::A_BYTES];
  __shared__ __align__(32) unsigned char s_vraw[Ly::V_BYTES];
  __shared__ double s_u[kMaxL];
  __shared__ double s_row_r[64], s_row_w[64], s_row_m[64], s_row_den[64];
  TIn* const s_k = reinterpret_cast<TIn*>(s_araw);
  double* const s_b = reinterpret_cast<double*>(s_araw);
  double* const s_ct = reinterpret_cast<double*>(s_araw);
  TIn* const s_vt = reinterpret_cast<TIn*>(s_vraw);
  double* const s_tot = reinterpret_cast<double*>(s_vraw);

  const int NQT = p.L > 64 ? p.L / 64 : 1;  // chunks below 64 rows: one tile
  const TileIdx ti = xcd_tile();
  int bid = ti.x;
  const int qt = bid % NQT;
  bid /= NQT;
  const int c = bid % p.Nc;
  const int bh = bid / p.Nc;
  const int vt = ti.y;
  const int S = p.S, DV = p.DV, L = p.L, Nc = p.Nc;
  const int t0 = c * L, Lc = min(L, S - t0), row0 = qt * 64;
  if (row0 >= Lc) return;
  const int kend = min(row0 + 64, Lc);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, l16 = lane & 15;
  const double scale = (double)p.scale;
  const TIn* Q = static_cast<const TIn*>(p.Q) + ((size_t)bh * S + t0) * DK;
  const TIn* K = static_cast<const TIn*>(p.K) + ((size_t)bh * S + t0) * DK;
  const TIn* V = static_cast<const TIn*>(p.V) + ((size_t)bh * S + t0) * DV + vt * TV;
  const float* ig = p.i_pre + (size_t)bh * S + t0;
  const float* fg = p.f_pre + (size_t)bh * S + t0;
  const double* Cst = reinterpret_cast<const double*>(p.C_states) + ((size_t)bh * (Nc + 1) + c) * DK * DV + vt * TV;
  const double* nst = reinterpret_cast<const double*>(p.n_states) + ((size_t)bh * (Nc + 1) + c) * DK;

  // ---- gates over chunk positions [0, kend): b, u = src - b, and per row of
  // the tile the exponent offset r, the inter-term weight w and m
  {
    double b[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int pos = 4 * tid + e;
      b[e] = pos < kend ? log_sigmoid_d((double)fg[pos]) : 0.0;
    }
    block_scan4_d<false>(b, s_tot);
    double u[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int pos = 4 * tid + e;
      if (pos < kend) {
        const double it = (double)ig[pos];
        u[e] = (SIG ? log_sigmoid_d(it) : it) - b[e];
        s_b[pos] = b[e];
        s_u[pos] = u[e];
      } else {
        u[e] = -INFINITY;
      }
    }
    if constexpr (!SIG) {
      block_scan4_d<true>(u, s_tot);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int pos = 4 * tid + e;
        if (pos >= row0 && pos < kend) s_row_m[pos - row0] = u[e];  // prefix max for now
      }
    }
    __syncthreads();
    if (tid < 64) {
      const int pos = row0 + tid;
      if (pos < kend) {
        if constexpr (SIG) {
          s_row_r[tid] = s_b[pos];
          s_row_w[tid] = exp(s_b[pos]);
          s_row_m[tid] = 0.0;
        } else {
          const double Mp = reinterpret_cast<const double*>(p.m_states)[(size_t)bh * (Nc + 1) + c];
          const double mx = fmax(Mp, s_row_m[tid]);
          s_row_r[tid] = -mx;
          s_row_w[tid] = exp(Mp - mx);
          s_row_m[tid] = s_b[pos] + mx;
        }
      } else {
        s_row_r[tid] = 0.0;
        s_row_w[tid] = 0.0;
        s_row_m[tid] = 0.0;
      }
    }
    __syncthreads();  // s_b and s_tot are free again
  }

  // ---- the query tile (rows past the chunk stage zeros)
  for (int idx = tid; idx < 64 * (DK / VN); idx += 256) {
    const int r = idx / (DK / VN), cc = (idx % (DK / VN)) * VN;
    uint4 x = make_uint4(0u, 0u, 0u, 0u);
    if (row0 + r < Lc) x = *reinterpret_cast<const uint4*>(Q + (size_t)(row0 + r) * DK + cc);
    *reinterpret_cast<uint4*>(s_q + r * Ly::LDI + cc) = x;
  }

  // ---- inter-chunk term acc = Q C over 16-row blocks of the state
  double4_t acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = double4_t{0.0, 0.0, 0.0, 0.0};
  const TIn* const qrow = s_q + (16 * w + l16) * Ly::LDI + 4 * g;
  for (int k0 = 0; k0 < DK; k0 += 16) {
    for (int idx = tid; idx < 16 * TV; idx += 256) {
      const int kr = idx / TV, col = idx % TV;
      s_ct[col * Ly::LDC + kr] = Cst[(size_t)(k0 + kr) * DV + col];
    }
    __syncthreads();
    double qa[4];
    lds4<TIn>(qrow + k0, qa);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const double4_t cv = *reinterpret_cast<const double4_t*>(s_ct + (16 * cb + l16) * Ly::LDC + 4 * g);
#pragma unroll
      for (int s = 0; s < 4; ++s) acc[cb] = mma_f64(qa[s], cv[s], acc[cb]);
    }
    __syncthreads();
  }
  // normaliser contribution of the state: s w q . n per row
  if constexpr (!SIG) {
    if (tid < 64) {
      double d = 0.0;
      for (int k0 = 0; k0 < DK; k0 += 4) {
        double q4[4];
        lds4<TIn>(s_q + tid * Ly::LDI + k0, q4);
#pragma unroll
        for (int e = 0; e < 4; ++e) d = fma(q4[e], nst[k0 + e], d);
      }
      s_row_den[tid] = d * s_row_w[tid] * scale;
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const double wr = s_row_w[16 * w + 4 * r + g] * scale;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[cb][r] *= wr;
  }

  // ---- intra-chunk term over key tiles of 64 keys
  const int tau = row0 + 16 * w + l16;  // this lane's row in the score blocks
  const double rr = s_row_r[16 * w + l16];
  double dsum = 0.0;
  const int ntiles = (kend + 63) / 64;
  for (int j = 0; j < ntiles; ++j) {
    const int s0 = j * 64;
    __syncthreads();  // the previous tile's reads (and the state blocks') are done
    for (int idx = tid; idx < 64 * (DK / VN); idx += 256) {
      const int r = idx / (DK / VN), cc = (idx % (DK / VN)) * VN;
      uint4 x = make_uint4(0u, 0u, 0u, 0u);
      if (s0 + r < Lc) x = *reinterpret_cast<const uint4*>(K + (size_t)(s0 + r) * DK + cc);
      *reinterpret_cast<uint4*>(s_k + r * Ly::LDI + cc) = x;
    }
    for (int idx = tid; idx < 64 * (TV / VN); idx += 256) {
      const int r = idx / (TV / VN), cc = (idx % (TV / VN)) * VN;
      TIn x[VN];
      if (s0 + r < Lc) {
        *reinterpret_cast<uint4*>(x) = *reinterpret_cast<const uint4*>(V + (size_t)(s0 + r) * DV + cc);
      } else {
        *reinterpret_cast<uint4*>(x) = make_uint4(0u, 0u, 0u, 0u);
      }
      // key 16 a + 4 r' + g goes to position 16 a + 4 g + r'
      const int pos = (r & ~15) | ((r & 3) << 2) | ((r >> 2) & 3);
#pragma unroll
      for (int e = 0; e < VN; ++e) s_vt[(cc + e) * Ly::LDV + pos] = x[e];
    }
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int key0 = s0 + 16 * kb;
      if (key0 > row0 + 16 * w + 15 || key0 >= kend) continue;  // wave-uniform: all zero
      // S^T for keys key0 .. + 15 against this wave's 16 rows
      // two accumulation chains (even and odd 16-deep steps), summed after
      double4_t st = double4_t{0.0, 0.0, 0.0, 0.0}, st1 = st;
      const TIn* const krow = s_k + (16 * kb + l16) * Ly::LDI + 4 * g;
#pragma unroll 2
      for (int k0 = 0; k0 < DK; k0 += 32) {
        double ka[4], qb[4], ka1[4], qb1[4];
        lds4<TIn>(krow + k0, ka);
        lds4<TIn>(qrow + k0, qb);
        lds4<TIn>(krow + k0 + 16, ka1);
        lds4<TIn>(qrow + k0 + 16, qb1);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          st = mma_f64(ka[s], qb[s], st);
          st1 = mma_f64(ka1[s], qb1[s], st1);
        }
      }
      st += st1;
      // P for keys key0 + 4 r + g of row tau (causal; rows past the chunk zero)
      double pr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = key0 + 4 * r + g;
        pr[r] = (key <= tau && tau < kend) ? scale * st[r] * exp(rr + s_u[key]) : 0.0;
        dsum += pr[r];
      }
      // acc += P V: product r takes key key0 + 4 r + g in slot g
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        double vb[4];
        lds4<TIn>(s_vt + (16 * cb + l16) * Ly::LDV + 16 * kb + 4 * g, vb);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[cb] = mma_f64(pr[r], vb[r], acc[cb]);
      }
    }
  }

  // ---- normaliser per row, then H
  dsum += __shfl_xor(dsum, 16, 64);
  dsum += __shfl_xor(dsum, 32, 64);
  __syncthreads();
  if constexpr (!SIG) {
    if (g == 0) s_row_den[16 * w + l16] += dsum;
  }
  __syncthreads();
  float* Hf = static_cast<float*>(p.H);
  uint16_t* Hb = static_cast<uint16_t*>(p.H);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 16 * w + 4 * r + g, t = row0 + row;
    if (t >= Lc) continue;
    double norm = 1.0;
    if constexpr (!SIG) norm = fmax(fabs(s_row_den[row]), exp(-s_row_m[row])) + (double)p.eps;
    const double inv = 1.0 / norm;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const double h = acc[cb][r] * inv;
      const size_t off = ((size_t)bh * S + t0 + t) * DV + vt * TV + 16 * cb + l16;
      if (p.h_bf16) Hb[off] = f32_to_bf16((float)h);
      else Hf[off] = (float)h;
    }
  }
  if constexpr (!SIG) {
    if (vt == 0 && tid < 64 && row0 + tid < Lc) {
      const size_t ro = (size_t)bh * S + t0 + row0 + tid;
      if (p.m_rows) p.m_rows[ro] = (float)s_row_m[tid];
      if (p.den_rows) p.den_rows[ro] = (float)s_row_den[tid];
    }
  }
}

template <typename TIn, bool SIG>
hipError_t launch_states_t(const StatesParams& p, hipStream_t stream) {
  // 32-column tiles when 64-column ones leave fewer than two workgroups per CU
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if ((long long)p.BH * (p.DK / 64) * (p.DV / 64) < 2LL * cus) {
    dim3 grid(p.BH, p.DK / 64, p.DV / 32);
    hipLaunchKernelGGL((states_f64m_kernel<TIn, SIG, 32>), grid, dim3(256), 0, stream, p);
  } else {
    dim3 grid(p.BH, p.DK / 64, p.DV / 64);
    hipLaunchKernelGGL((states_f64m_kernel<TIn, SIG, 64>), grid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

template <typename TIn, bool SIG, int DK, int TV>
hipError_t launch_hintra_t(const HintraParams& p, hipStream_t stream) {
  dim3 grid((unsigned)(p.BH * p.Nc * (p.L > 64 ? p.L / 64 : 1)), p.DV / TV);
  hipLaunchKernelGGL((hintra_f64m_kernel<TIn, SIG, DK, TV>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <typename TIn, bool SIG, int DK>
hipError_t launch_hintra_tv(const HintraParams& p, hipStream_t stream) {
  // float32 tiles of 256-wide rows leave LDS room for 64 columns only
  constexpr bool wide_ok = !(std::is_same<TIn, float>::value && DK == 256);
  if constexpr (wide_ok)
    if (p.DV % 128 == 0) return launch_hintra_t<TIn, SIG, DK, 128>(p, stream);
  return launch_hintra_t<TIn, SIG, DK, 64>(p, stream);
}

template <typename TIn, bool SIG>
hipError_t launch_hintra_dk(const HintraParams& p, hipStream_t stream) {
  switch (p.DK) {
    case 64: return launch_hintra_tv<TIn, SIG, 64>(p, stream);
    case 128: return launch_hintra_tv<TIn, SIG, 128>(p, stream);
    case 256: return launch_hintra_tv<TIn, SIG, 256>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool hintra_f64m_supported(int DK) { return DK == 64 || DK == 128 || DK == 256; }

hipError_t launch_states_f64(const StatesParams& p, bool bf16_inputs, bool sig, hipStream_t stream) {
  if (bf16_inputs) return sig ? launch_states_t<bf16_t, true>(p, stream) : launch_states_t<bf16_t, false>(p, stream);
  return sig ? launch_states_t<float, true>(p, stream) : launch_states_t<float, false>(p, stream);
}

hipError_t launch_hintra_f64m(const HintraParams& p, bool bf16_inputs, bool sig, hipStream_t stream) {
  if (bf16_inputs) return sig ? launch_hintra_dk<bf16_t, true>(p, stream) : launch_hintra_dk<bf16_t, false>(p, stream);
  return sig ? launch_hintra_dk<float, true>(p, stream) : launch_hintra_dk<float, false>(p, stream);
}

}  // namespace mlstm
