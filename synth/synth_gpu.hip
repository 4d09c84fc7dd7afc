/*
 * Device copy of the counter-based generator in synth.c, for filling large
 * calibration stand-ins (X, G) directly in device memory.  It evaluates the
 * same per-element formulas in the same order (mix64, keys, uniforms,
 * Box-Muller cosine branch, Student t(4) chi-square part, f64 -> f32 -> bf16
 * rounding to nearest even); the per-column factors (outlier scale, gradient
 * channel scale) come from synth_col_factors on the host, so the two
 * generators can differ only where a device libm result (log, cos) differs
 * from the host's in the last bit and that difference survives the rounding
 * to the output type.  Tests that compare against host-generated data check
 * the columns they use for bit-identity.  Like synth.c it holds none of the
 * quantizer's arithmetic.  Built with -ffp-contract=off.
 */
#include <hip/hip_runtime.h>
#include <stdint.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

namespace {

enum { SYN_NORMAL = 0, SYN_ACT_NORMAL = 1, SYN_ACT_T4 = 2, SYN_GRAD_LOGNORMAL = 3, SYN_INT = 4,
       SYN_ACT_T4_DRIFT = 5 };
enum { OUT_F64 = 0, OUT_F32 = 1, OUT_BF16 = 2 };

__host__ __device__ inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

__host__ __device__ inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed) ^ ((stream + 1) * GAMMA));
}

__device__ inline uint64_t u64_at(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GAMMA); }

__device__ inline double unif_at(uint64_t key, uint64_t i) {
  return ((double)(u64_at(key, i) >> 11) + 0.5) * 0x1.0p-53;
}

__device__ inline double normal_at(uint64_t key, uint64_t e) {
  const double two_pi = 6.283185307179586476925286766559;
  double u1 = unif_at(key, 2 * e), u2 = unif_at(key, 2 * e + 1);
  return sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
}

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

struct Keys {
  uint64_t k0, k1, k3, k6, k7;
};

__global__ void __launch_bounds__(256) synth_fill(int kind, Keys k, int64_t rows, int64_t cols, double p1,
                                                  const double* __restrict__ colf, int out_dtype,
                                                  void* __restrict__ out, int64_t ld) {
  const int64_t total = rows * cols;
  const int64_t ip1 = (int64_t)p1;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * 256) {
    const int64_t r = idx / cols, c = idx % cols;
    const uint64_t e = (uint64_t)idx;
    double v;
    switch (kind) {
      case SYN_NORMAL: v = p1 * normal_at(k.k0, e); break;
      case SYN_ACT_NORMAL: v = normal_at(k.k1, e) * colf[c]; break;
      case SYN_ACT_T4: {
        const double z = normal_at(k.k1, e);
        const double ua = unif_at(k.k6, 2 * e), ub = unif_at(k.k6, 2 * e + 1);
        v = z * sqrt(2.0 / -log(ua * ub)) * colf[c];
        break;
      }
      case SYN_GRAD_LOGNORMAL: v = normal_at(k.k3, e) * colf[c]; break;
      case SYN_ACT_T4_DRIFT: {
        const double z = normal_at(k.k1, e);
        const double ua = unif_at(k.k6, 2 * e), ub = unif_at(k.k6, 2 * e + 1);
        v = (z * sqrt(2.0 / -log(ua * ub)) + p1 * normal_at(k.k7, e)) * colf[c];
        break;
      }
      default: v = (double)((int64_t)(u64_at(k.k1, e) % (uint64_t)(2 * ip1 + 1)) - ip1); break;
    }
    const int64_t o = r * ld + c;
    if (out_dtype == OUT_F64) static_cast<double*>(out)[o] = v;
    else if (out_dtype == OUT_F32) static_cast<float*>(out)[o] = (float)v;
    else static_cast<uint16_t*>(out)[o] = f32_to_bf16_rne((float)v);
  }
}

}  // namespace

/* Whole rows x cols matrix of `kind` into device memory `out` (leading
 * dimension ld elements); colf: device array of the cols column factors.
 * Returns 0, 1 on bad arguments, 3 on a HIP error. */
extern "C" int synth_matrix_dev(int kind, uint64_t seed, int64_t rows, int64_t cols, double p1,
                                const double* colf, int out_dtype, void* out, int64_t ld, void* stream) {
  if (rows < 0 || cols < 0 || ld < cols || (rows > 0 && cols > 0 && (!out || !colf))) return 1;
  if (out_dtype < OUT_F64 || out_dtype > OUT_BF16 || kind < SYN_NORMAL || kind > SYN_ACT_T4_DRIFT) return 1;
  if (rows == 0 || cols == 0) return 0;
  Keys k{stream_key(seed, 0), stream_key(seed, 1), stream_key(seed, 3), stream_key(seed, 6),
         stream_key(seed, 7)};
  const int64_t total = rows * cols;
  const unsigned grid = (unsigned)((total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536);
  hipLaunchKernelGGL(synth_fill, dim3(grid), dim3(256), 0, (hipStream_t)stream, kind, k, rows, cols, p1,
                     colf, out_dtype, out, ld);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}
