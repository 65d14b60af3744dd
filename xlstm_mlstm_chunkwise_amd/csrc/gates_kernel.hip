// Per-position gate terms of the chunkwise form, computed once per chunk and
// shared by both stages of the wide-tile path.
//
// Within chunk c (positions t0 .. t0 + Lc - 1, local index tau) the
// chunkwise-parallel mLSTM ("Tiled Flash Linear Attention: More Efficient
// Linear RNN and xLSTM Kernels", abstract; the mLSTM recurrence of "xLSTM: the
// NX-AI repository behind the extended LSTM architecture", section
// "Exponential gating, matrix memory, and why the kernels decide everything")
// needs, with lf = log sigmoid(f) and i~ = i (exp gate) or log sigmoid(i)
// (sig gate):
//   b_tau  = lf_0 + ... + lf_tau          in-chunk inclusive cumulative sum
//   u_tau  = i~_tau - b_tau               input term seen from the chunk start
//   pm_tau = max(u_0, ..., u_tau)         (exp gate) running maximum of u
// They are stored in log2 units (times log2 e), the units of the hardware
// exponential the consumers use:
//   gb2[bh][t], gu2[bh][t], gpm2[bh][t]   float32, t = absolute position.
// From them, the state update of a chunk is
//   M' = b_last + max(M, pm_last),  weight of step tau = e^{b_last + u_tau - M'}
// and the intra-chunk decay between key sigma and query tau <= sigma' is
//   e^{u_sigma - max(M, pm_tau)}   relative to the stabiliser m_tau = b_tau + max(M, pm_tau).
// One workgroup per (head, chunk); 256 threads x 4 positions cover L <= 1024.
#include "device_common.h"
#include "kernels.h"

namespace mlstm {
namespace {

template <bool SIG>
__global__ __launch_bounds__(256) void gates_kernel(const GatesParams p) {
  __shared__ float s_red[4];
  const int c = blockIdx.x % p.Nc;
  const int bh = blockIdx.x / p.Nc;
  const int t0 = c * p.L;
  const int Lc = min(p.L, p.S - t0);
  const size_t base = (size_t)bh * p.S + t0;
  const int tid = threadIdx.x;

  float f[4], in[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int pos = 4 * tid + e;
    f[e] = pos < Lc ? p.f_pre[base + pos] : 0.0f;
    in[e] = pos < Lc ? p.i_pre[base + pos] : 0.0f;
  }
  float b[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) b[e] = 4 * tid + e < Lc ? log_sigmoid(f[e]) : 0.0f;
  block_scan4<false, 4>(b, s_red);
  float u[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int pos = 4 * tid + e;
    if (pos < Lc) {
      u[e] = ((SIG ? log_sigmoid(in[e]) : in[e]) - b[e]) * kLog2e;
      p.gb2[base + pos] = b[e] * kLog2e;
      p.gu2[base + pos] = u[e];
    } else {
      u[e] = -INFINITY;
    }
  }
  if constexpr (!SIG) {
    block_scan4<true, 4>(u, s_red);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int pos = 4 * tid + e;
      if (pos < Lc) p.gpm2[base + pos] = u[e];
    }
  }
}

}  // namespace

hipError_t launch_gates(const GatesParams& p, bool sig, hipStream_t stream) {
  if (p.S == 0 || p.BH == 0) return hipSuccess;
  const dim3 grid((unsigned)(p.BH * p.Nc));
  if (sig) hipLaunchKernelGGL(gates_kernel<true>, grid, dim3(256), 0, stream, p);
  else hipLaunchKernelGGL(gates_kernel<false>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mlstm
