// Float64 evaluation of both stages of the chunkwise mLSTM forward pass
// (precision mode MLSTM_PREC_F64), for inputs whose rows are too
// ill-conditioned for float32 accumulation.
//
// The arithmetic is the chunkwise form used by the other kernels (TFLA
// abstract: chunkwise-parallel recurrence with intra-chunk tiling; mLSTM
// normaliser and max-state), carried out entirely in fp64 on the vector
// ALUs: gate sums, exponentials, scores, contractions and the chunk states
// (kept in fp64 in the workspace).  Each thread owns a 4 x 4 register block;
// operands are staged through LDS in 64-wide tiles.
#include "device_common.h"
#include "tile_order.h"
#include "kernels.h"

namespace mlstm {
namespace {

constexpr int kMaxL = 1024;

__device__ __forceinline__ double log_sigmoid_d(double x) { return fmin(x, 0.0) - log1p(exp(-fabs(x))); }

template <typename TIn>
__device__ __forceinline__ double load_in(const TIn* p, size_t i);
template <>
__device__ __forceinline__ double load_in<float>(const float* p, size_t i) {
  return static_cast<double>(p[i]);
}
template <>
__device__ __forceinline__ double load_in<bf16_t>(const bf16_t* p, size_t i) {
  return static_cast<double>(bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i]));
}

// Block-wide inclusive scan (sum or max) of 4 doubles per thread; 256 threads.
template <bool IS_MAX>
__device__ void block_scan4_d(double (&v)[4], double* tot) {
  const double ident = IS_MAX ? -INFINITY : 0.0;
  for (int e = 1; e < 4; ++e) v[e] = IS_MAX ? fmax(v[e - 1], v[e]) : v[e - 1] + v[e];
  const int tid = threadIdx.x;
  tot[tid] = v[3];
  __syncthreads();
  // Hillis-Steele over the 256 thread totals (double buffer in tot[0..511]).
  double* a = tot;
  double* b = tot + 256;
  for (int off = 1; off < 256; off <<= 1) {
    const double x = a[tid];
    const double y = tid >= off ? a[tid - off] : ident;
    b[tid] = IS_MAX ? fmax(x, y) : x + y;
    __syncthreads();
    double* t = a;
    a = b;
    b = t;
  }
  const double pre = tid > 0 ? a[tid - 1] : ident;
  __syncthreads();
  for (int e = 0; e < 4; ++e) v[e] = IS_MAX ? fmax(pre, v[e]) : pre + v[e];
}

__device__ double block_max_d(double x, double* scratch) {
  const int tid = threadIdx.x;
  scratch[tid] = x;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) scratch[tid] = fmax(scratch[tid], scratch[tid + off]);
    __syncthreads();
  }
  const double r = scratch[0];
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------------------
// Stage one: 64 x 64 tile of C per workgroup, thread t owns rows 4*(t/16)..+3
// and columns 4*(t%16)..+3 of the tile.

template <typename TIn, bool SIG>
__global__ __launch_bounds__(256) void states_f64_kernel(const StatesParams p) {
  __shared__ double s_w[kMaxL];
  __shared__ double s_tot[512];
  __shared__ double s_g;
  __shared__ double s_k[32][65];
  __shared__ double s_vv[32][65];

  const int bh = blockIdx.x, kt = blockIdx.y, vt = blockIdx.z;
  const int tid = threadIdx.x, kq = tid >> 4, vq = tid & 15;
  const int S = p.S, DK = p.DK, DV = p.DV, L = p.L, Nc = p.Nc;
  const TIn* K = static_cast<const TIn*>(p.K) + (size_t)bh * S * DK;
  const TIn* V = static_cast<const TIn*>(p.V) + (size_t)bh * S * DV;
  const float* ig = p.i_pre + (size_t)bh * S;
  const float* fg = p.f_pre + (size_t)bh * S;
  const bool own_n = !SIG && vt == 0;
  double* Cs = reinterpret_cast<double*>(p.C_states);
  double* ns = reinterpret_cast<double*>(p.n_states);
  double* ms = reinterpret_cast<double*>(p.m_states);

  double acc[4][4];
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j) {
      const int kr = kt * 64 + 4 * kq + i, vc = vt * 64 + 4 * vq + j;
      acc[i][j] = p.C0 ? (double)p.C0[(size_t)bh * DK * DV + (size_t)kr * DV + vc] : 0.0;
    }
  double nreg = 0.0;
  if (own_n && tid < 64 && p.n0) nreg = p.n0[(size_t)bh * DK + kt * 64 + tid];
  double M = (!SIG && p.m0) ? (double)p.m0[bh] : 0.0;

  for (int c = 0; c <= Nc; ++c) {
    double* Cst = Cs + ((size_t)bh * (Nc + 1) + c) * DK * DV;
    for (int i = 0; i < 4; ++i)
      for (int j = 0; j < 4; ++j) Cst[(size_t)(kt * 64 + 4 * kq + i) * DV + vt * 64 + 4 * vq + j] = acc[i][j];
    if (own_n && tid < 64) ns[((size_t)bh * (Nc + 1) + c) * DK + kt * 64 + tid] = nreg;
    if (!SIG && kt == 0 && vt == 0 && tid == 0) ms[(size_t)bh * (Nc + 1) + c] = M;
    if (c == Nc) break;

    const int t0 = c * L, Lc = min(L, S - t0);
    double b[4];
    for (int e = 0; e < 4; ++e) {
      const int pos = 4 * tid + e;
      b[e] = pos < Lc ? log_sigmoid_d((double)fg[t0 + pos]) : 0.0;
    }
    block_scan4_d<false>(b, s_tot);
    for (int e = 0; e < 4; ++e)
      if (4 * tid + e == Lc - 1) s_g = b[e];
    __syncthreads();
    const double g = s_g;
    double a[4], amax = -INFINITY;
    for (int e = 0; e < 4; ++e) {
      const int pos = 4 * tid + e;
      if (pos < Lc) {
        const double it = (double)ig[t0 + pos];
        a[e] = g - b[e] + (SIG ? log_sigmoid_d(it) : it);
        amax = fmax(amax, a[e]);
      } else {
        a[e] = -INFINITY;
      }
    }
    double decay;
    if constexpr (SIG) {
      decay = exp(g);
      for (int e = 0; e < 4; ++e) s_w[4 * tid + e] = (4 * tid + e < Lc) ? exp(a[e]) : 0.0;
    } else {
      amax = block_max_d(amax, s_tot);
      const double Mn = fmax(g + M, amax);
      decay = exp(g + M - Mn);
      for (int e = 0; e < 4; ++e) s_w[4 * tid + e] = (4 * tid + e < Lc) ? exp(a[e] - Mn) : 0.0;
      M = Mn;
    }
    __syncthreads();
    for (int i = 0; i < 4; ++i)
      for (int j = 0; j < 4; ++j) acc[i][j] *= decay;
    nreg *= decay;

    for (int tb = 0; tb < Lc; tb += 32) {
      for (int idx = tid; idx < 32 * 64; idx += 256) {
        const int t = idx >> 6, col = idx & 63;
        const bool ok = tb + t < Lc;
        s_k[t][col] = ok ? load_in<TIn>(K, (size_t)(t0 + tb + t) * DK + kt * 64 + col) * s_w[tb + t] : 0.0;
        s_vv[t][col] = ok ? load_in<TIn>(V, (size_t)(t0 + tb + t) * DV + vt * 64 + col) : 0.0;
      }
      __syncthreads();
      if (own_n && tid < 64) {
        double sacc = 0.0;
        for (int t = 0; t < 32; ++t) sacc += s_k[t][tid];
        nreg += sacc;
      }
#pragma unroll 2
      for (int t = 0; t < 32; ++t) {
        double kk[4], vv[4];
        for (int i = 0; i < 4; ++i) kk[i] = s_k[t][4 * kq + i];
        for (int j = 0; j < 4; ++j) vv[j] = s_vv[t][4 * vq + j];
        for (int i = 0; i < 4; ++i)
          for (int j = 0; j < 4; ++j) acc[i][j] = fma(kk[i], vv[j], acc[i][j]);
      }
      __syncthreads();
    }
  }
  if (p.C_out)
    for (int i = 0; i < 4; ++i)
      for (int j = 0; j < 4; ++j)
        p.C_out[(size_t)bh * DK * DV + (size_t)(kt * 64 + 4 * kq + i) * DV + vt * 64 + 4 * vq + j] =
            (float)acc[i][j];
  if (own_n && p.n_out && tid < 64) p.n_out[(size_t)bh * DK + kt * 64 + tid] = (float)nreg;
  if (!SIG && p.m_out && kt == 0 && vt == 0 && tid == 0) p.m_out[bh] = (float)M;
}

// ---------------------------------------------------------------------------
// Stage two: 64 rows x 64 columns of H per workgroup; thread t owns rows
// 4*(t/16)..+3 and columns (or keys) 4*(t%16)..+3.

template <typename TIn, bool SIG>
__global__ __launch_bounds__(256) void hintra_f64_kernel(const HintraParams p) {
  __shared__ double s_b[kMaxL];
  __shared__ double s_u[kMaxL];
  __shared__ double s_tot[512];
  __shared__ double s_q[64][33];
  __shared__ double s_x[64][33];  // key rows [sigma][k], or state block [k][v] as [v][k]
  __shared__ double s_pv[64][65]; // P tile [tau][sigma], then values [sigma][v]
  __shared__ double s_vt[64][65];
  __shared__ double s_row_r[64], s_row_w[64], s_row_m[64], s_row_den[64];

  const int NQT = p.L > 64 ? p.L / 64 : 1;  // chunks below 64 rows: one tile
  const TileIdx ti = xcd_tile();
  int bid = ti.x;
  const int qt = bid % NQT;
  bid /= NQT;
  const int c = bid % p.Nc;
  const int bh = bid / p.Nc;
  const int vt = ti.y;
  const int S = p.S, DK = p.DK, DV = p.DV, L = p.L, Nc = p.Nc;
  const int t0 = c * L, Lc = min(L, S - t0), row0 = qt * 64;
  if (row0 >= Lc) return;
  const int kend = min(row0 + 64, Lc);
  const int tid = threadIdx.x, rq = tid >> 4, cq = tid & 15;
  const double scale = (double)p.scale;
  const TIn* Q = static_cast<const TIn*>(p.Q) + ((size_t)bh * S + t0) * DK;
  const TIn* K = static_cast<const TIn*>(p.K) + ((size_t)bh * S + t0) * DK;
  const TIn* V = static_cast<const TIn*>(p.V) + ((size_t)bh * S + t0) * DV;
  const float* ig = p.i_pre + (size_t)bh * S + t0;
  const float* fg = p.f_pre + (size_t)bh * S + t0;
  const double* Cst = reinterpret_cast<const double*>(p.C_states) + ((size_t)bh * (Nc + 1) + c) * DK * DV;
  const double* nst = reinterpret_cast<const double*>(p.n_states) + ((size_t)bh * (Nc + 1) + c) * DK;

  // gates
  {
    double b[4];
    for (int e = 0; e < 4; ++e) {
      const int pos = 4 * tid + e;
      b[e] = pos < kend ? log_sigmoid_d((double)fg[pos]) : 0.0;
    }
    block_scan4_d<false>(b, s_tot);
    double u[4];
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
    __syncthreads();
  }

  double acc[4][4] = {};
  double den_part = 0.0;  // for row 4*rq + (cq & 3) after the final reduction
  // inter-chunk term, k blocks of 32
  for (int kb = 0; kb < DK; kb += 32) {
    for (int idx = tid; idx < 64 * 32; idx += 256) {
      const int r = idx >> 5, k = idx & 31;
      s_q[r][k] = (row0 + r < Lc) ? load_in<TIn>(Q, (size_t)(row0 + r) * DK + kb + k) : 0.0;
      const int v = idx >> 5;  // 64 columns x 32 k
      s_x[v][k] = Cst[(size_t)(kb + k) * DV + vt * 64 + v];
    }
    __syncthreads();
#pragma unroll 2
    for (int k = 0; k < 32; ++k) {
      double qa[4], cb[4];
      for (int i = 0; i < 4; ++i) qa[i] = s_q[4 * rq + i][k];
      for (int j = 0; j < 4; ++j) cb[j] = s_x[4 * cq + j][k];
      for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j) acc[i][j] = fma(qa[i], cb[j], acc[i][j]);
    }
    if constexpr (!SIG) {
      if (tid < 64) {
        double d = 0.0;
#pragma unroll 4
        for (int k = 0; k < 32; ++k) d = fma(s_q[tid][k], nst[kb + k], d);
        s_row_den[tid] = (kb == 0 ? 0.0 : s_row_den[tid]) + d;
      }
    }
    __syncthreads();
  }
  for (int i = 0; i < 4; ++i) {
    const double w = s_row_w[4 * rq + i] * scale;
    for (int j = 0; j < 4; ++j) acc[i][j] *= w;
  }
  if constexpr (!SIG) {
    __syncthreads();
    if (tid < 64) s_row_den[tid] *= s_row_w[tid] * scale;
    __syncthreads();
  }

  // intra-chunk term, key tiles of 64
  double dsum[4] = {0.0, 0.0, 0.0, 0.0};
  const int ntiles = (kend + 63) / 64;
  for (int j = 0; j < ntiles; ++j) {
    const int s0 = j * 64;
    double sacc[4][4] = {};
    for (int kb = 0; kb < DK; kb += 32) {
      for (int idx = tid; idx < 64 * 32; idx += 256) {
        const int r = idx >> 5, k = idx & 31;
        s_q[r][k] = (row0 + r < Lc) ? load_in<TIn>(Q, (size_t)(row0 + r) * DK + kb + k) : 0.0;
        s_x[r][k] = (s0 + r < Lc) ? load_in<TIn>(K, (size_t)(s0 + r) * DK + kb + k) : 0.0;
      }
      __syncthreads();
#pragma unroll 2
      for (int k = 0; k < 32; ++k) {
        double qa[4], ka[4];
        for (int i = 0; i < 4; ++i) qa[i] = s_q[4 * rq + i][k];
        for (int jj = 0; jj < 4; ++jj) ka[jj] = s_x[4 * cq + jj][k];
        for (int i = 0; i < 4; ++i)
          for (int jj = 0; jj < 4; ++jj) sacc[i][jj] = fma(qa[i], ka[jj], sacc[i][jj]);
      }
      __syncthreads();
    }
    for (int i = 0; i < 4; ++i) {
      const int tau = row0 + 4 * rq + i;
      const double rr = s_row_r[4 * rq + i];
      for (int jj = 0; jj < 4; ++jj) {
        const int sg = s0 + 4 * cq + jj;
        double val = 0.0;
        if (sg <= tau && tau < kend) val = scale * sacc[i][jj] * exp(rr + s_u[sg]);
        s_pv[4 * rq + i][4 * cq + jj] = val;
        dsum[i] += val;
      }
    }
    for (int idx = tid; idx < 64 * 64; idx += 256) {
      const int sg = idx >> 6, v = idx & 63;
      s_vt[sg][v] = (s0 + sg < Lc) ? load_in<TIn>(V, (size_t)(s0 + sg) * DV + vt * 64 + v) : 0.0;
    }
    __syncthreads();
#pragma unroll 2
    for (int sg = 0; sg < 64; ++sg) {
      double pa[4], vb[4];
      for (int i = 0; i < 4; ++i) pa[i] = s_pv[4 * rq + i][sg];
      for (int jj = 0; jj < 4; ++jj) vb[jj] = s_vt[sg][4 * cq + jj];
      for (int i = 0; i < 4; ++i)
        for (int jj = 0; jj < 4; ++jj) acc[i][jj] = fma(pa[i], vb[jj], acc[i][jj]);
    }
    __syncthreads();
  }
  // row sums of P: reduce dsum over the 16 threads (cq) sharing a row block
  for (int i = 0; i < 4; ++i) {
    double x = dsum[i];
    for (int off = 8; off > 0; off >>= 1) x += __shfl_xor(x, off, 16);
    dsum[i] = x;
  }
  if constexpr (!SIG) {
    if (cq == 0)
      for (int i = 0; i < 4; ++i) s_row_den[4 * rq + i] += dsum[i];
  }
  __syncthreads();
  (void)den_part;
  float* Hf = static_cast<float*>(p.H);
  uint16_t* Hb = static_cast<uint16_t*>(p.H);
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * rq + i, t = row0 + row;
    if (t >= Lc) continue;
    double norm = 1.0;
    if constexpr (!SIG) norm = fmax(fabs(s_row_den[row]), exp(-s_row_m[row])) + (double)p.eps;
    for (int jj = 0; jj < 4; ++jj) {
      const double h = acc[i][jj] / norm;
      const size_t off = ((size_t)bh * S + t0 + t) * DV + vt * 64 + 4 * cq + jj;
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

__global__ __launch_bounds__(256) void narrow_f64_kernel(const double* src, float* dst, long long n) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = (float)src[i];
}

}  // namespace

hipError_t launch_states_f64(const StatesParams& p, bool bf16_inputs, bool sig, hipStream_t stream) {
  dim3 grid(p.BH, p.DK / 64, p.DV / 64);
  if (bf16_inputs) {
    if (sig) hipLaunchKernelGGL((states_f64_kernel<bf16_t, true>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((states_f64_kernel<bf16_t, false>), grid, dim3(256), 0, stream, p);
  } else {
    if (sig) hipLaunchKernelGGL((states_f64_kernel<float, true>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((states_f64_kernel<float, false>), grid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_hintra_f64(const HintraParams& p, bool bf16_inputs, bool sig, hipStream_t stream) {
  dim3 grid((unsigned)(p.BH * p.Nc * (p.L > 64 ? p.L / 64 : 1)), p.DV / 64);
  if (bf16_inputs) {
    if (sig) hipLaunchKernelGGL((hintra_f64_kernel<bf16_t, true>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((hintra_f64_kernel<bf16_t, false>), grid, dim3(256), 0, stream, p);
  } else {
    if (sig) hipLaunchKernelGGL((hintra_f64_kernel<float, true>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((hintra_f64_kernel<float, false>), grid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_narrow_f64(const void* src, float* dst, long long n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(narrow_f64_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     static_cast<const double*>(src), dst, n);
  return hipGetLastError();
}

}  // namespace mlstm
