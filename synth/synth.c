/*
 * Seeded synthetic inputs for the KronQ sublayer quantization path.
 *
 * This module generates the calibration stand-ins (activations X, output
 * gradients G), the weights W and the random sign vectors of the randomized
 * Hadamard transforms.  It holds none of the quantizer's arithmetic; both the
 * GPU library's tests and the CPU oracle draw their inputs from here, so the
 * two sides always see the same bytes.
 *
 * Generator (counter based, so any sub-block of a matrix can be produced on its
 * own and the result does not depend on the thread count):
 *   mix(z)        : the splitmix64 output function (Steele, Lea, Flood 2014)
 *   key(seed, s)  : mix(mix(seed) ^ ((s + 1) * GAMMA))
 *   u64(key, i)   : mix(key + (i + 1) * GAMMA)
 *   unif(key, i)  : ((u64 >> 11) + 0.5) * 2^-53, strictly inside (0, 1)
 *   normal(key,e) : Box-Muller, cosine branch, from unif(key,2e), unif(key,2e+1)
 *   t4(e)         : normal(k1,e) * sqrt(2 / -ln(unif(k2,2e) * unif(k2,2e+1)))
 *                   (Student t with 4 degrees of freedom: chi2_4 / 4 =
 *                   -ln(u_a u_b) / 2; variance 2)
 * Element (r, c) of a logical rows x cols matrix uses counter e = r * cols + c.
 * Streams: 0 weights, 1 activations, 2 outlier-channel choice, 3 gradient
 * noise, 4 gradient channel scales, 5 Hadamard signs, 6 chi-square part of t4,
 * 7 input drift.
 * Values are produced in double and rounded to the output type: f32 by
 * round-to-nearest-even; bf16 by f64 -> f32 -> bf16, each step nearest-even.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

enum { SYN_NORMAL = 0, SYN_ACT_NORMAL = 1, SYN_ACT_T4 = 2, SYN_GRAD_LOGNORMAL = 3, SYN_INT = 4,
       SYN_ACT_T4_DRIFT = 5 };
enum { OUT_F64 = 0, OUT_F32 = 1, OUT_BF16 = 2 };

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed) ^ ((stream + 1) * GAMMA));
}

static inline uint64_t u64_at(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GAMMA); }

static inline double unif_at(uint64_t key, uint64_t i) {
  return ((double)(u64_at(key, i) >> 11) + 0.5) * 0x1.0p-53;
}

static inline double normal_at(uint64_t key, uint64_t e) {
  const double two_pi = 6.283185307179586476925286766559;
  double u1 = unif_at(key, 2 * e), u2 = unif_at(key, 2 * e + 1);
  return sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

uint64_t synth_mix64(uint64_t z) { return mix64(z); }
uint64_t synth_stream_key(uint64_t seed, uint64_t stream) { return stream_key(seed, stream); }

/* Partial Fisher-Yates over 0..n-1 with stream 2: the first k entries. */
int synth_outlier_channels(uint64_t seed, int64_t n, int64_t k, int64_t* out) {
  if (n <= 0 || k < 0 || k > n || (k > 0 && !out)) return 1;
  int64_t* idx = (int64_t*)malloc(sizeof(int64_t) * (size_t)n);
  if (!idx) return 2;
  for (int64_t i = 0; i < n; ++i) idx[i] = i;
  uint64_t key = stream_key(seed, 2);
  for (int64_t i = 0; i < k; ++i) {
    int64_t j = i + (int64_t)(u64_at(key, (uint64_t)i) % (uint64_t)(n - i));
    int64_t t = idx[i]; idx[i] = idx[j]; idx[j] = t;
    out[i] = idx[i];
  }
  free(idx);
  return 0;
}

/* +-1 signs with stream 5 of `seed`: sign = top bit of u64 set ? -1 : +1. */
int synth_signs(uint64_t seed, int64_t n, float* out) {
  if (n < 0 || (n > 0 && !out)) return 1;
  uint64_t key = stream_key(seed, 5);
  for (int64_t i = 0; i < n; ++i) out[i] = (u64_at(key, (uint64_t)i) >> 63) ? -1.0f : 1.0f;
  return 0;
}

/*
 * Column factors of columns [c0, c0+nc): out_factor on the listed outlier
 * columns of the activation kinds, exp(p1 * normal(stream 4, column)) for the
 * gradient kind, 1 otherwise.
 */
int synth_col_factors(int kind, uint64_t seed, int64_t c0, int64_t nc, double p1,
                      const int64_t* outliers, int64_t n_out, double out_factor, double* colf) {
  if (c0 < 0 || nc < 0 || (nc > 0 && !colf)) return 1;
  for (int64_t c = 0; c < nc; ++c) colf[c] = 1.0;
  if (kind == SYN_ACT_NORMAL || kind == SYN_ACT_T4 || kind == SYN_ACT_T4_DRIFT) {
    for (int64_t o = 0; o < n_out; ++o) {
      int64_t ch = outliers[o];
      if (ch >= c0 && ch < c0 + nc) colf[ch - c0] = out_factor;
    }
  } else if (kind == SYN_GRAD_LOGNORMAL) {
    uint64_t k4 = stream_key(seed, 4);
    for (int64_t c = 0; c < nc; ++c) colf[c] = exp(p1 * normal_at(k4, (uint64_t)(c0 + c)));
  }
  return 0;
}

/*
 * Fill block [r0, r0+nr) x [c0, c0+nc) of a logical rows x cols matrix.
 *   kind SYN_NORMAL         : p1 * normal(stream 0)
 *   kind SYN_ACT_NORMAL     : normal(stream 1) * channel factor
 *   kind SYN_ACT_T4         : t4(stream 1, stream 6) * channel factor
 *   kind SYN_GRAD_LOGNORMAL : normal(stream 3) * exp(p1 * normal(stream 4, column))
 *   kind SYN_INT            : integer uniform in [-p1, p1] (stream 1)
 *   kind SYN_ACT_T4_DRIFT   : (t4(stream 1, stream 6) + p1 * normal(stream 7)) *
 *                             channel factor: the SYN_ACT_T4 matrix of the same
 *                             seed before rounding, plus a drift of relative
 *                             size p1 (the full-precision model's inputs next to
 *                             the inputs of a partly quantized model)
 * The channel factor is out_factor for the columns listed in outliers[0..n_out),
 * 1 elsewhere.  out is row-major with leading dimension ld (elements).
 */
int synth_matrix(int kind, uint64_t seed, int64_t rows, int64_t cols, int64_t r0, int64_t nr,
                 int64_t c0, int64_t nc, double p1, const int64_t* outliers, int64_t n_out,
                 double out_factor, int out_dtype, void* out, int64_t ld) {
  if (rows < 0 || cols < 0 || r0 < 0 || c0 < 0 || nr < 0 || nc < 0) return 1;
  if (r0 + nr > rows || c0 + nc > cols || ld < nc || (nr > 0 && nc > 0 && !out)) return 1;
  if (out_dtype < OUT_F64 || out_dtype > OUT_BF16) return 1;
  if (kind < SYN_NORMAL || kind > SYN_ACT_T4_DRIFT) return 1;
  double* colf = (double*)malloc(sizeof(double) * (size_t)(nc > 0 ? nc : 1));
  if (!colf) return 2;
  synth_col_factors(kind, seed, c0, nc, p1, outliers, n_out, out_factor, colf);
  uint64_t k0 = stream_key(seed, 0), k1 = stream_key(seed, 1), k3 = stream_key(seed, 3),
           k6 = stream_key(seed, 6), k7 = stream_key(seed, 7);
  int64_t ip1 = (int64_t)p1;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < nr; ++r) {
    for (int64_t c = 0; c < nc; ++c) {
      uint64_t e = (uint64_t)(r0 + r) * (uint64_t)cols + (uint64_t)(c0 + c);
      double v;
      switch (kind) {
        case SYN_NORMAL: v = p1 * normal_at(k0, e); break;
        case SYN_ACT_NORMAL: v = normal_at(k1, e) * colf[c]; break;
        case SYN_ACT_T4: {
          double z = normal_at(k1, e);
          double ua = unif_at(k6, 2 * e), ub = unif_at(k6, 2 * e + 1);
          v = z * sqrt(2.0 / -log(ua * ub)) * colf[c];
          break;
        }
        case SYN_GRAD_LOGNORMAL: v = normal_at(k3, e) * colf[c]; break;
        case SYN_ACT_T4_DRIFT: {
          double z = normal_at(k1, e);
          double ua = unif_at(k6, 2 * e), ub = unif_at(k6, 2 * e + 1);
          v = (z * sqrt(2.0 / -log(ua * ub)) + p1 * normal_at(k7, e)) * colf[c];
          break;
        }
        default: v = (double)((int64_t)(u64_at(k1, e) % (uint64_t)(2 * ip1 + 1)) - ip1); break;
      }
      int64_t o = r * ld + c;
      if (out_dtype == OUT_F64) ((double*)out)[o] = v;
      else if (out_dtype == OUT_F32) ((float*)out)[o] = (float)v;
      else ((uint16_t*)out)[o] = f32_to_bf16_rne((float)v);
    }
  }
  free(colf);
  return 0;
}
