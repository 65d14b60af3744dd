// Packed chunk states -> float32 row-major (n_states, DK, DV).
//
// The wide kernels keep each state as bf16 hi + lo fragments of 16 rows x 32
// columns (device_common.h, packed chunk-state layout): lane l of a fragment
// holds column 32 nb + l % 32 and, in its eight slots e, rows
// 16 kk + (e < 4 ? 0 : 8) + 4 (l / 32) + e % 4.  One thread per fragment lane
// reads its 16-byte hi and lo pieces and writes the eight values; the 32
// lanes of a half-wave write 128 contiguous bytes of a row each time.  The
// int16-coded form has one 16-byte piece of eight codes per fragment lane
// (fragment f = kk * (DV / 32) + nb at codes 512 f) and one scale per
// fragment.
#include "device_common.h"
#include "kernels.h"

namespace mlstm {
namespace {

template <bool CODES>
__global__ __launch_bounds__(256) void unpack_states_kernel(const uint16_t* __restrict__ P,
                                                            const float* __restrict__ scales, float* __restrict__ C,
                                                            long long nfrag_lanes, int DK, int DV) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= nfrag_lanes) return;
  const int lane = (int)(i & 63);
  const long long frag = i >> 6;                 // (state, kk, nb)
  const int nfr = (DK / 16) * (DV / 32);         // fragments per state
  const long long st = frag / nfr;
  const int f = (int)(frag % nfr), kk = f / (DV / 32), nb = f % (DV / 32);
  float* dst = C + st * (long long)DK * DV + (size_t)(32 * nb + (lane & 31));
  if constexpr (CODES) {
    const uint4 u = *reinterpret_cast<const uint4*>(P + frag * 512 + lane * 8);
    const float sc = scales[frag];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int code = e & 1 ? (int)w[e >> 1] >> 16 : (int)(w[e >> 1] << 16) >> 16;
      const int k = 16 * kk + (e < 4 ? 0 : 8) + 4 * (lane >> 5) + (e & 3);
      dst[(size_t)k * DV] = (float)code * sc;
    }
    return;
  }
  const uint16_t* src = P + st * (long long)DK * DV * 2;
  const uint4 hi = *reinterpret_cast<const uint4*>(src + pack_frag_offset(kk, nb, 0, DV) + lane * 8);
  const uint4 lo = *reinterpret_cast<const uint4*>(src + pack_frag_offset(kk, nb, 1, DV) + lane * 8);
  const uint32_t hw[4] = {hi.x, hi.y, hi.z, hi.w}, lw[4] = {lo.x, lo.y, lo.z, lo.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t h = e & 1 ? hw[e >> 1] & 0xffff0000u : hw[e >> 1] << 16;
    const uint32_t l = e & 1 ? lw[e >> 1] & 0xffff0000u : lw[e >> 1] << 16;
    const int k = 16 * kk + (e < 4 ? 0 : 8) + 4 * (lane >> 5) + (e & 3);
    dst[(size_t)k * DV] = __uint_as_float(h) + __uint_as_float(l);
  }
}

}  // namespace

hipError_t launch_unpack_states(const void* packed, float* C, long long n_states, int DK, int DV,
                                hipStream_t stream, const float* scales) {
  const long long lanes = n_states * (DK / 16) * (DV / 32) * 64;
  if (lanes == 0) return hipSuccess;
  const dim3 grid((unsigned)((lanes + 255) / 256));
  if (scales)
    hipLaunchKernelGGL(unpack_states_kernel<true>, grid, dim3(256), 0, stream, static_cast<const uint16_t*>(packed),
                       scales, C, lanes, DK, DV);
  else
    hipLaunchKernelGGL(unpack_states_kernel<false>, grid, dim3(256), 0, stream,
                       static_cast<const uint16_t*>(packed), scales, C, lanes, DK, DV);
  return hipGetLastError();
}

}  // namespace mlstm
