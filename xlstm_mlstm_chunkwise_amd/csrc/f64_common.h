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

// Block-wide inclusive scan (sum or max) of 4 doubles per thread; 256 threads.
template <bool IS_MAX>
__device__ inline void block_scan4_d(double (&v)[4], double* tot) {
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

__device__ inline double block_max_d(double x, double* scratch) {
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

}  // namespace f64
}  // namespace mlstm
