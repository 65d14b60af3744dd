// Float64 helpers shared by the fp64 kernels of precision mode MLSTM_PREC_F64
// (vector-unit kernels in f64_kernels.hip, matrix-core kernels in
// f64_mfma_kernels.hip): log-sigmoid, input widening and block scans of 256
// threads in double precision.
#pragma once
#include "device_common.h"

namespace mlstm {
namespace f64 {

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

// Block-wide inclusive scan (sum or max) of 4 doubles per thread; 256
// threads (4 waves).  Each thread scans its 4 values, each wave scans its 64
// thread totals with lane shuffles, and the waves' totals go through LDS
// (`tot`, at least 4 doubles): two barriers in all.
template <bool IS_MAX>
__device__ inline void block_scan4_d(double (&v)[4], double* tot) {
  const double ident = IS_MAX ? -INFINITY : 0.0;
  for (int e = 1; e < 4; ++e) v[e] = IS_MAX ? fmax(v[e - 1], v[e]) : v[e - 1] + v[e];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double x = v[3];
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(x, off, 64);
    if (lane >= off) x = IS_MAX ? fmax(x, y) : x + y;
  }
  if (lane == 63) tot[wave] = x;
  __syncthreads();
  double pre = ident;
  for (int w = 0; w < wave; ++w) pre = IS_MAX ? fmax(pre, tot[w]) : pre + tot[w];
  double ex = __shfl_up(x, 1, 64);  // this wave's total before this thread
  if (lane == 0) ex = ident;
  pre = IS_MAX ? fmax(pre, ex) : pre + ex;
  __syncthreads();  // tot is free again
  for (int e = 0; e < 4; ++e) v[e] = IS_MAX ? fmax(pre, v[e]) : pre + v[e];
}

// Maximum over the block (256 threads): lane shuffles within each wave, the
// four wave maxima through LDS (`scratch`, at least 4 doubles).
__device__ inline double block_max_d(double x, double* scratch) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmax(x, __shfl_xor(x, off, 64));
  if (lane == 0) scratch[wave] = x;
  __syncthreads();
  const double r = fmax(fmax(scratch[0], scratch[1]), fmax(scratch[2], scratch[3]));
  __syncthreads();
  return r;
}

}  // namespace f64
}  // namespace mlstm
