// Sensitivity score s = tr(H_X) tr(H_G) of a sublayer, computed on the
// post-BiIP factors (hyper.ai summary of the KronQ paper, Method, Eq. 14).
// One workgroup per factor sums its diagonal in fp64: each thread accumulates a
// strided slice, then the wavefront reduces with cross-lane shuffles and the
// waves meet in LDS; a final single lane forms the product.
#include "kronq_internal.h"

namespace kronq {
namespace {

constexpr int TT = 256;

__device__ inline double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__global__ void __launch_bounds__(TT) trace_kernel(const float* HX, int64_t n, int64_t ldhx,
                                                   const float* HG, int64_t m, int64_t ldhg,
                                                   double* out3) {
  __shared__ double part[2][TT / 64];
  const float* H = blockIdx.x == 0 ? HX : HG;
  const int64_t d = blockIdx.x == 0 ? n : m;
  const int64_t ld = blockIdx.x == 0 ? ldhx : ldhg;
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < d; i += TT) acc += (double)H[i * ld + i];
  acc = wave_sum(acc);
  if ((threadIdx.x & 63) == 0) part[0][threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int w = 0; w < TT / 64; ++w) t += part[0][w];
    out3[blockIdx.x] = t;
  }
}

__global__ void trace_product(double* out3) {
  if (threadIdx.x == 0) out3[2] = out3[0] * out3[1];
}

}  // namespace

kronq_status trace_launch(const float* HX, int64_t n, int64_t ldhx, const float* HG, int64_t m,
                          int64_t ldhg, double* out3, hipStream_t s) {
  hipLaunchKernelGGL(trace_kernel, dim3(2), dim3(TT), 0, s, HX, n, ldhx, HG, m, ldhg, out3);
  KQ_LAUNCHED("trace_kernel");
  hipLaunchKernelGGL(trace_product, dim3(1), dim3(64), 0, s, out3);
  KQ_LAUNCHED("trace_product");
  return KRONQ_OK;
}

}  // namespace kronq
