// Float64 evaluation of the intra-chunk stage of the chunkwise mLSTM forward
// pass (precision mode MLSTM_PREC_F64) on the vector ALUs, for the key widths
// the matrix-core kernels (f64_mfma_kernels.hip) do not take (512), and the
// narrowing of the fp64 chunk states to float32.
//
// The arithmetic is the chunkwise form used by the other kernels (TFLA
// abstract: chunkwise-parallel recurrence with intra-chunk tiling; mLSTM
// normaliser and max-state), carried out entirely in fp64: gate sums,
// exponentials, scores and contractions, against chunk states kept in fp64
// in the workspace.  Each thread owns a 4 x 4 register block; operands are
// staged through LDS in 64-wide tiles.
#include "device_common.h"
#include "f64_common.h"
#include "tile_order.h"
#include "kernels.h"

namespace mlstm {
namespace {

using namespace f64;

// ---------------------------------------------------------------------------
// Stage two: 64 rows x 64 columns of H per workgroup; thread t owns rows
// 4*(t/16)..+3 and columns (or keys) 4*(t%16)..+3.

template <typename TIn, bool SIG>
__global__ __launch_bounds__(256) void hintra_f64_kernel(const HintraParams p) {
  __shared__ double s_b[kMaxL];
  __shared__ double s_u[kMaxL];
  __shared__ double s_tot[4];  // wave totals of the block scans
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

hipError_t launch_hintra_f64(const HintraParams& p, bool bf16_inputs, bool sig, hipStream_t stream) {
  if (hintra_f64m_supported(p.DK)) return launch_hintra_f64m(p, bf16_inputs, sig, stream);
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
