// Host half of libkronq: argument validation, workspace checks, dispatch to the
// kernel launchers, and the host-only bit allocator.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>
#include <algorithm>

#include "kronq_internal.h"

namespace kronq {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

kronq_status fail(kronq_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

kronq_status hip_fail(hipError_t e, const char* what) {
  set_error("%s: %s (%d)", what, hipGetErrorString(e), (int)e);
  return KRONQ_EHIP;
}

static bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

static bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

static kronq_status check_had(const kronq_had* h, int64_t dim, const char* side) {
  if (!h) return fail(KRONQ_EINVAL, "%s Hadamard spec is NULL", side);
  if (h->dim != dim)
    return fail(KRONQ_EINVAL, "%s Hadamard dim %lld != matrix dimension %lld", side,
                (long long)h->dim, (long long)dim);
  if (!pow2(h->block) || h->block > 32768 || dim % h->block)
    return fail(KRONQ_EINVAL, "%s Hadamard block %lld must be a power of two <= 32768 dividing %lld",
                side, (long long)h->block, (long long)dim);
  if (!h->signs && h->block != 1)
    return fail(KRONQ_EINVAL, "%s Hadamard signs are NULL (allowed only with block 1: identity)", side);
  return KRONQ_OK;
}

// Workspace size and alignment (16 bytes: the kernels read and write their
// parts of it with 16-byte vector accesses).
static kronq_status check_ws(const char* fn, const void* ws, size_t ws_bytes, size_t need,
                             bool always) {
  if (ws_bytes < need || ((need || always) && !ws))
    return fail(KRONQ_EWORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  if (ws && !aligned(ws, 16)) return fail(KRONQ_EINVAL, "%s: workspace must be 16-byte aligned", fn);
  return KRONQ_OK;
}

// Argument checks of the individual calls (no workspace).
static kronq_status check_gram(const void* A, int32_t dtype, int64_t N, int64_t d, int64_t lda,
                               const float* H, int64_t ldh, float scale, float beta) {
  if (!A || !H) return fail(KRONQ_EINVAL, "kronq_gram: NULL pointer");
  if (dtype != KRONQ_F32 && dtype != KRONQ_BF16)
    return fail(KRONQ_EINVAL, "kronq_gram: dtype %d", (int)dtype);
  if (N < 1 || d < 1) return fail(KRONQ_EINVAL, "kronq_gram: N=%lld d=%lld", (long long)N, (long long)d);
  if (lda < d || ldh < d) return fail(KRONQ_EINVAL, "kronq_gram: leading dimension below d");
  if (!aligned(A, 16) || !aligned(H, 16))
    return fail(KRONQ_EINVAL, "kronq_gram: A and H must be 16-byte aligned");
  if ((dtype == KRONQ_BF16 && lda % 8) || (dtype == KRONQ_F32 && lda % 4))
    return fail(KRONQ_EINVAL, "kronq_gram: lda must be a multiple of 16 bytes");
  if (!std::isfinite(scale) || !std::isfinite(beta))
    return fail(KRONQ_EINVAL, "kronq_gram: scale/beta not finite");
  return KRONQ_OK;
}

static kronq_status check_biip(const float* W, int64_t m, int64_t n, int64_t ldw, const float* HX,
                               int64_t ldhx, const float* HG, int64_t ldhg,
                               const kronq_had* in_side, const kronq_had* out_side, float alpha) {
  if (!W) return fail(KRONQ_EINVAL, "kronq_biip_rotate: W is NULL");
  if (m < 1 || n < 1 || ldw < n) return fail(KRONQ_EINVAL, "kronq_biip_rotate: bad W shape");
  if (HX && ldhx < n) return fail(KRONQ_EINVAL, "kronq_biip_rotate: ldhx < n");
  if (HG && ldhg < m) return fail(KRONQ_EINVAL, "kronq_biip_rotate: ldhg < m");
  if (!std::isfinite(alpha)) return fail(KRONQ_EINVAL, "kronq_biip_rotate: alpha not finite");
  if (alpha != 0.0f && !HG)
    return fail(KRONQ_EINVAL, "kronq_biip_rotate: the output rescale needs HG");
  kronq_status st = check_had(in_side, n, "input-side");
  if (st) return st;
  return check_had(out_side, m, "output-side");
}

static kronq_status check_chol(const float* H, int64_t n, int64_t ldh, float lambda,
                               const int32_t* perm, const float* R, int64_t ldr,
                               const int64_t* info) {
  if (!H || !R || !perm || !info) return fail(KRONQ_EINVAL, "kronq_chol_inv: NULL pointer");
  if (n < 1 || ldh < n || ldr < n) return fail(KRONQ_EINVAL, "kronq_chol_inv: bad shape");
  if (!(lambda >= 0.0f) || !std::isfinite(lambda))
    return fail(KRONQ_EINVAL, "kronq_chol_inv: lambda must be finite and >= 0");
  return KRONQ_OK;
}

static kronq_status check_gptq(const float* W, int64_t m, int64_t n, int64_t ldw, const float* R,
                               int64_t ldr, const kronq_qcfg* q, const uint8_t* codes,
                               const float* scales, const float* zeros, const float* What) {
  if (!W || !R || !q || !codes || !scales || !zeros)
    return fail(KRONQ_EINVAL, "kronq_gptq_quantize: NULL pointer");
  if (m < 1 || n < 1 || ldw < n || ldr < n)
    return fail(KRONQ_EINVAL, "kronq_gptq_quantize: bad shape");
  if (!aligned(R, 16) || ldr % 4 != 0)
    return fail(KRONQ_EINVAL, "kronq_gptq_quantize: R must be 16-byte aligned with ldr a multiple of 4");
  if (q->bits < 1 || q->bits > 8)
    return fail(KRONQ_EINVAL, "kronq_gptq_quantize: bits %d outside 1..8", (int)q->bits);
  if (q->group > 0 && n % q->group)
    return fail(KRONQ_EINVAL, "kronq_gptq_quantize: group %d does not divide n", (int)q->group);
  if (What == W && ldw != n)
    return fail(KRONQ_EINVAL, "kronq_gptq_quantize: What may alias W only when ldw == n");
  return KRONQ_OK;
}

// Argument checks shared by the two decode entry points (no workspace).
static kronq_status check_decode(const char* fn, const uint8_t* codes, int64_t m, int64_t n,
                                 int64_t ldp, const kronq_qcfg* q, const float* scales,
                                 const float* zeros, const int32_t* perm, const kronq_had* in_side,
                                 const kronq_had* out_side, const float* x, const float* y) {
  if (!codes || !q || !scales || !zeros || !x || !y) return fail(KRONQ_EINVAL, "%s: NULL pointer", fn);
  if (q->bits < 1 || q->bits > 8)
    return fail(KRONQ_EINVAL, "%s: bits %d outside 1..8", fn, (int)q->bits);
  if (m < 1 || n < 1 || n > INT32_MAX || m > INT32_MAX) return fail(KRONQ_EINVAL, "%s: bad shape", fn);
  if (ldp < decode_row_bytes(n, q->bits) || ldp % 16 || !aligned(codes, 16))
    return fail(KRONQ_EINVAL,
                "%s: codes must be 16-byte aligned with ldp a multiple of 16 covering a row (%lld "
                "bytes)", fn, (long long)decode_row_bytes(n, q->bits));
  if (q->group > 0) {
    if (n % q->group) return fail(KRONQ_EINVAL, "%s: group does not divide n", fn);
    if (q->group % 64)
      return fail(KRONQ_EUNSUPPORTED, "%s: group %d is not a multiple of 64", fn, (int)q->group);
  }
  if (perm && n > 32768)
    return fail(KRONQ_EUNSUPPORTED, "%s: codes in processing order need n <= 32768 (got %lld)", fn,
                (long long)n);
  kronq_status st = check_had(in_side, n, "input-side");
  if (st) return st;
  return check_had(out_side, m, "output-side");
}

}  // namespace kronq

using namespace kronq;

extern "C" {

const char* kronq_status_string(kronq_status s) {
  switch (s) {
    case KRONQ_OK: return "ok";
    case KRONQ_EINVAL: return "invalid argument";
    case KRONQ_ENOTPD: return "matrix not positive definite";
    case KRONQ_EHIP: return "HIP runtime error";
    case KRONQ_EWORKSPACE: return "workspace too small";
    case KRONQ_EUNSUPPORTED: return "unsupported";
    case KRONQ_ENUMERIC: return "non-finite value";
    case KRONQ_ENOMEM: return "request exceeds a fixed device buffer";
    default: return "unknown status";
  }
}

const char* kronq_last_error(void) { return g_err; }

int32_t kronq_version(void) { return 1; }

// The sign draw: splitmix64's finalizer over a counter with the golden-ratio
// increment, keyed by the seed (stream 5 of the seed's key sequence).
static uint64_t sm64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

kronq_status kronq_signs(uint64_t seed, int64_t n, float* out_host) {
  if (n < 0 || (n > 0 && !out_host)) return fail(KRONQ_EINVAL, "kronq_signs: n=%lld out=%p",
                                                 (long long)n, (void*)out_host);
  const uint64_t g = 0x9E3779B97F4A7C15ULL;
  const uint64_t key = sm64_mix(sm64_mix(seed) ^ (6ULL * g));
  for (int64_t i = 0; i < n; ++i)
    out_host[i] = (sm64_mix(key + (uint64_t)(i + 1) * g) >> 63) ? -1.0f : 1.0f;
  return KRONQ_OK;
}

kronq_status kronq_check_finite(const float* A, int64_t rows, int64_t cols, int64_t ld,
                                int32_t* flag_dev, void* stream) {
  if (!flag_dev) return fail(KRONQ_EINVAL, "kronq_check_finite: flag is NULL");
  if (rows < 0 || cols < 0) return fail(KRONQ_EINVAL, "kronq_check_finite: negative shape");
  if (rows > 0 && cols > 0 && (!A || ld < cols))
    return fail(KRONQ_EINVAL, "kronq_check_finite: NULL matrix or ld < cols");
  return finite_launch(A, rows, cols, ld, flag_dev, (hipStream_t)stream);
}

size_t kronq_gram_ws(int64_t N, int64_t d, int32_t dtype) {
  if (N < 1 || d < 1 || (dtype != KRONQ_F32 && dtype != KRONQ_BF16)) return 0;
  return gram_ws_bytes(N, d, dtype);
}

kronq_status kronq_gram(const void* A, int32_t dtype, int64_t N, int64_t d, int64_t lda, float* H,
                        int64_t ldh, float scale, float beta, void* ws, size_t ws_bytes,
                        void* stream) {
  kronq_status st = check_gram(A, dtype, N, d, lda, H, ldh, scale, beta);
  if (st) return st;
  size_t need = gram_ws_bytes(N, d, dtype);
  st = check_ws("kronq_gram", ws, ws_bytes, need, false);
  if (st) return st;
  return gram_launch(A, dtype, N, d, lda, H, ldh, scale, beta, ws, ws_bytes, (hipStream_t)stream);
}

size_t kronq_biip_ws(int64_t m, int64_t n) {
  if (m < 1 || n < 1) return 0;
  return biip_ws_bytes(m, n);
}

kronq_status kronq_biip_rotate(float* W, int64_t m, int64_t n, int64_t ldw, float* HX,
                               int64_t ldhx, float* HG, int64_t ldhg, const kronq_had* in_side,
                               const kronq_had* out_side, float alpha, float* sg, void* ws,
                               size_t ws_bytes, void* stream) {
  kronq_status st = check_biip(W, m, n, ldw, HX, ldhx, HG, ldhg, in_side, out_side, alpha);
  if (st) return st;
  size_t need = biip_ws_bytes(m, n);
  st = check_ws("kronq_biip_rotate", ws, ws_bytes, need, false);
  if (st) return st;
  return biip_launch(W, m, n, ldw, HX, ldhx, HG, ldhg, *in_side, *out_side, alpha, sg, ws, ws_bytes,
                     (hipStream_t)stream);
}

size_t kronq_incoherence_ws(int64_t n) {
  if (n < 1 || n > 32768) return 0;
  return eig_ws_bytes(n);
}

kronq_status kronq_incoherence(const float* H, int64_t n, int64_t ldh, double tol, int32_t max_sweeps,
                               double* mu, double* evals, double* Q, int64_t ldq, int32_t* sweeps,
                               void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "kronq_incoherence";
  if (!H || !mu) return fail(KRONQ_EINVAL, "%s: H or mu is NULL", fn);
  if (n < 1 || n > 32768 || ldh < n) return fail(KRONQ_EINVAL, "%s: bad H shape", fn);
  if (Q && ldq < n) return fail(KRONQ_EINVAL, "%s: ldq < n", fn);
  if (!(tol >= 1e-15 && tol <= 1e-2)) return fail(KRONQ_EINVAL, "%s: tol outside [1e-15, 1e-2]", fn);
  if (max_sweeps < 1 || max_sweeps > 100) return fail(KRONQ_EINVAL, "%s: max_sweeps outside 1..100", fn);
  kronq_status st = check_ws(fn, ws, ws_bytes, eig_ws_bytes(n), true);
  if (st) return st;
  return eig_launch(H, n, ldh, tol, max_sweeps, mu, evals, Q, ldq, sweeps, ws, (hipStream_t)stream);
}

size_t kronq_biip_sx_ws(int64_t m, int64_t n) {
  if (m < 1 || n < 1) return 0;
  return biip_sx_ws_bytes(m, n);
}

kronq_status kronq_biip_rotate_sx(float* W, int64_t m, int64_t n, int64_t ldw, float* HX,
                                  int64_t ldhx, float* HG, int64_t ldhg, const kronq_had* in_side,
                                  const kronq_had* out_side, float alpha, float alpha_x, float* sg,
                                  float* sx, int32_t sx_given, void* ws, size_t ws_bytes,
                                  void* stream) {
  const char* fn = "kronq_biip_rotate_sx";
  if (!W && !HX && !HG) return fail(KRONQ_EINVAL, "%s: W, HX and HG are all NULL", fn);
  if (m < 1 || n < 1 || (W && ldw < n)) return fail(KRONQ_EINVAL, "%s: bad W shape", fn);
  if (HX && ldhx < n) return fail(KRONQ_EINVAL, "%s: ldhx < n", fn);
  if (HG && ldhg < m) return fail(KRONQ_EINVAL, "%s: ldhg < m", fn);
  if (!std::isfinite(alpha) || !std::isfinite(alpha_x))
    return fail(KRONQ_EINVAL, "%s: alpha or alpha_x not finite", fn);
  if (alpha != 0.0f && !HG) return fail(KRONQ_EINVAL, "%s: the output rescale needs HG", fn);
  if (sx_given != 0 && sx_given != 1) return fail(KRONQ_EINVAL, "%s: sx_given must be 0 or 1", fn);
  if (sx_given && !sx) return fail(KRONQ_EINVAL, "%s: sx_given but sx is NULL", fn);
  if (!sx_given && alpha_x != 0.0f && !HX)
    return fail(KRONQ_EINVAL, "%s: the input rescale needs HX (or a given sx)", fn);
  kronq_status st = check_had(in_side, n, "input-side");
  if (st) return st;
  st = check_had(out_side, m, "output-side");
  if (st) return st;
  st = check_ws(fn, ws, ws_bytes, biip_sx_ws_bytes(m, n), true);
  if (st) return st;
  return biip_launch(W, m, n, ldw, HX, ldhx, HG, ldhg, *in_side, *out_side, alpha, sg, ws, ws_bytes,
                     (hipStream_t)stream, true, alpha_x, sx_given ? sx : nullptr,
                     sx_given ? nullptr : sx);
}

size_t kronq_biip_unrotate_sx_ws(int64_t m, int64_t n) {
  if (m < 1 || n < 1) return 0;
  return unrotate_sx_ws_bytes(m, n);
}

kronq_status kronq_biip_unrotate_sx(float* W, int64_t m, int64_t n, int64_t ldw,
                                    const kronq_had* in_side, const kronq_had* out_side,
                                    const float* sg, const float* sx, void* ws, size_t ws_bytes,
                                    void* stream) {
  const char* fn = "kronq_biip_unrotate_sx";
  if (!W || !sx) return fail(KRONQ_EINVAL, "%s: W or sx is NULL", fn);
  if (m < 1 || n < 1 || ldw < n) return fail(KRONQ_EINVAL, "%s: bad W shape", fn);
  kronq_status st = check_had(in_side, n, "input-side");
  if (st) return st;
  st = check_had(out_side, m, "output-side");
  if (st) return st;
  st = check_ws(fn, ws, ws_bytes, unrotate_sx_ws_bytes(m, n), true);
  if (st) return st;
  return unrotate_sx_launch(W, m, n, ldw, *in_side, *out_side, sg, sx, ws, (hipStream_t)stream);
}

size_t kronq_biip_unrotate_ws(int64_t m, int64_t n) {
  if (m < 1 || n < 1) return 0;
  return unrotate_ws_bytes(m);
}

kronq_status kronq_biip_unrotate(float* W, int64_t m, int64_t n, int64_t ldw,
                                 const kronq_had* in_side, const kronq_had* out_side,
                                 const float* sg, void* ws, size_t ws_bytes, void* stream) {
  if (!W) return fail(KRONQ_EINVAL, "kronq_biip_unrotate: W is NULL");
  if (m < 1 || n < 1 || ldw < n) return fail(KRONQ_EINVAL, "kronq_biip_unrotate: bad W shape");
  kronq_status st = check_had(in_side, n, "input-side");
  if (st) return st;
  st = check_had(out_side, m, "output-side");
  if (st) return st;
  size_t need = unrotate_ws_bytes(m);
  st = check_ws("kronq_biip_unrotate", ws, ws_bytes, need, true);
  if (st) return st;
  return unrotate_launch(W, m, n, ldw, *in_side, *out_side, sg, ws, (hipStream_t)stream);
}

size_t kronq_chol_inv_ws(int64_t n) {
  if (n < 1) return 0;
  return chol_ws_bytes(n);
}

kronq_status kronq_chol_inv(const float* H, int64_t n, int64_t ldh, float lambda,
                            int32_t act_order, int32_t* perm, float* R, int64_t ldr,
                            int64_t* info, void* ws, size_t ws_bytes, void* stream) {
  if (info) *info = -1;
  kronq_status st = check_chol(H, n, ldh, lambda, perm, R, ldr, info);
  if (st) return st;
  size_t need = chol_ws_bytes(n);
  st = check_ws("kronq_chol_inv", ws, ws_bytes, need, false);
  if (st) return st;
  return chol_launch(H, n, ldh, lambda, act_order ? 1 : 0, perm, R, ldr, info, ws, ws_bytes,
                     (hipStream_t)stream);
}

size_t kronq_gptq_ws(int64_t m, int64_t n) {
  if (m < 1 || n < 1) return 0;
  return gptq_ws_bytes(m, n);
}

kronq_status kronq_gptq_quantize(const float* W, int64_t m, int64_t n, int64_t ldw,
                                 const float* R, int64_t ldr, const int32_t* perm,
                                 const kronq_qcfg* q, uint8_t* codes, float* scales,
                                 float* zeros, float* What, float* pre_round, double* row_loss,
                                 void* ws, size_t ws_bytes, void* stream) {
  kronq_status st = check_gptq(W, m, n, ldw, R, ldr, q, codes, scales, zeros, What);
  if (st) return st;
  size_t need = gptq_ws_bytes(m, n);
  st = check_ws("kronq_gptq_quantize", ws, ws_bytes, need, false);
  if (st) return st;
  return gptq_launch(W, m, n, ldw, R, ldr, perm, q->bits, q->group > 0 ? q->group : 0, codes,
                     scales, zeros, What, pre_round, row_loss, ws, ws_bytes, (hipStream_t)stream);
}

size_t kronq_gram_cross_ws(int64_t N, int64_t d) {
  if (N < 1 || d < 1) return 0;
  return gram_cross_ws_bytes(N, d);
}

kronq_status kronq_gram_cross(const void* A, const void* B, int64_t N, int64_t d, int64_t ld, float* C,
                              int64_t ldc, float scale, const float* sub, int64_t ldsub, void* ws,
                              size_t ws_bytes, void* stream) {
  if (!A || !B || !C) return fail(KRONQ_EINVAL, "kronq_gram_cross: NULL pointer");
  if (N < 1 || d < 1 || ld < d || ldc < d || (sub && ldsub < d))
    return fail(KRONQ_EINVAL, "kronq_gram_cross: bad shape");
  if (!aligned(A, 16) || !aligned(B, 16) || ld % 8 || !aligned(C, 16))
    return fail(KRONQ_EINVAL, "kronq_gram_cross: A, B and C must be 16-byte aligned, ld a multiple of 8");
  if (!std::isfinite(scale)) return fail(KRONQ_EINVAL, "kronq_gram_cross: scale not finite");
  if (d % 256 || N % 128)
    return fail(KRONQ_EUNSUPPORTED, "kronq_gram_cross: d (%lld) must be a multiple of 256 and N (%lld) "
                "of 128", (long long)d, (long long)N);
  if (!gram_pipeline_ld_ok(ld))
    return fail(KRONQ_EUNSUPPORTED, "kronq_gram_cross: ld (%lld) above 67108848", (long long)ld);
  const size_t need = gram_cross_ws_bytes(N, d);
  kronq_status st = check_ws("kronq_gram_cross", ws, ws_bytes, need, true);
  if (st) return st;
  return gram_cross_launch(A, B, N, d, ld, C, ldc, scale, 0.0f, sub, ldsub, ws, (hipStream_t)stream);
}

size_t kronq_drift_cross_ws(int64_t N, int64_t n) {
  if (N < 1 || n < 1) return 0;
  return drift_cross_ws_bytes(N, n);
}

kronq_status kronq_drift_cross(const void* Xfp, const void* X, int64_t N, int64_t n, int64_t ld, float* C,
                               int64_t ldc, void* ws, size_t ws_bytes, void* stream) {
  if (!Xfp || !X || !C) return fail(KRONQ_EINVAL, "kronq_drift_cross: NULL pointer");
  if (N < 1 || n < 1 || ld < n || ldc < n) return fail(KRONQ_EINVAL, "kronq_drift_cross: bad shape");
  if (!aligned(Xfp, 16) || !aligned(X, 16) || ld % 8 || !aligned(C, 16))
    return fail(KRONQ_EINVAL, "kronq_drift_cross: X, X_fp and C must be 16-byte aligned, ld a multiple of 8");
  if (n % 256 || N % 128)
    return fail(KRONQ_EUNSUPPORTED, "kronq_drift_cross: n (%lld) must be a multiple of 256 and N (%lld) "
                "of 128", (long long)n, (long long)N);
  if (!gram_pipeline_ld_ok(ld))
    return fail(KRONQ_EUNSUPPORTED, "kronq_drift_cross: ld (%lld) above 67108848", (long long)ld);
  kronq_status st = check_ws("kronq_drift_cross", ws, ws_bytes, drift_cross_ws_bytes(N, n), true);
  if (st) return st;
  return drift_cross_launch(Xfp, X, N, n, ld, C, ldc, ws, (hipStream_t)stream);
}

size_t kronq_gptaq_correction_ws(int64_t n) {
  if (n < 1) return 0;
  return gptaq_correction_ws_bytes(n);
}

kronq_status kronq_gptaq_correction(const float* C, int64_t n, int64_t ldc, const float* R, int64_t ldr,
                                    const int32_t* perm, float alpha, float* P, int64_t ldp, void* ws,
                                    size_t ws_bytes, void* stream) {
  if (!C || !R || !P) return fail(KRONQ_EINVAL, "kronq_gptaq_correction: NULL pointer");
  if (n < 1 || ldc < n || ldr < n || ldp < n) return fail(KRONQ_EINVAL, "kronq_gptaq_correction: bad shape");
  if (!std::isfinite(alpha)) return fail(KRONQ_EINVAL, "kronq_gptaq_correction: alpha not finite");
  kronq_status st = check_ws("kronq_gptaq_correction", ws, ws_bytes, gptaq_correction_ws_bytes(n), true);
  if (st) return st;
  return gptaq_correction_launch(C, n, ldc, R, ldr, perm, alpha, P, ldp, ws, (hipStream_t)stream);
}

size_t kronq_gptaq_ws(int64_t m, int64_t n) {
  if (m < 1 || n < 1) return 0;
  return align_up(gptq_ws_bytes(m, n), 256) + gptaq_shift_ws_bytes(m, n);
}

kronq_status kronq_gptaq_quantize(const float* W, int64_t m, int64_t n, int64_t ldw, const float* R,
                                  int64_t ldr, const int32_t* perm, const kronq_qcfg* q, const float* P,
                                  int64_t ldp, uint8_t* codes, float* scales, float* zeros, float* What,
                                  float* pre_round, double* row_loss, void* ws, size_t ws_bytes,
                                  void* stream) {
  kronq_status st = check_gptq(W, m, n, ldw, R, ldr, q, codes, scales, zeros, What);
  if (st) return st;
  if (!P || ldp < n) return fail(KRONQ_EINVAL, "kronq_gptaq_quantize: P is NULL or ldp < n");
  if (q->group > 0 && (128 % q->group != 0 || q->group % 8 != 0))
    return fail(KRONQ_EUNSUPPORTED, "kronq_gptaq_quantize: group %d must be a multiple of 8 dividing 128",
                (int)q->group);
  const size_t need = kronq_gptaq_ws(m, n);
  st = check_ws("kronq_gptaq_quantize", ws, ws_bytes, need, true);
  if (st) return st;
  const size_t off = align_up(gptq_ws_bytes(m, n), 256);
  float* W1 = reinterpret_cast<float*>(static_cast<char*>(ws) + off);
  float* X2 = reinterpret_cast<float*>(static_cast<char*>(ws) + off +
                                       align_up((size_t)m * (size_t)n * sizeof(float), 256));
  const int unit = q->group > 0 ? q->group : 128;
  st = gptaq_shift_launch(W, m, n, ldw, perm, P, ldp, unit, W1, X2, (hipStream_t)stream);
  if (st) return st;
  return gptq_launch(W, m, n, ldw, R, ldr, perm, q->bits, q->group > 0 ? q->group : 0, codes, scales,
                     zeros, What, pre_round, row_loss, ws, off, (hipStream_t)stream, W1, X2);
}

size_t kronq_weight_cv_ws(int64_t m, int64_t n) {
  if (m < 1 || n < 1) return 0;
  return cv_ws_bytes(m, n);
}

kronq_status kronq_weight_cv(const float* W, int64_t m, int64_t n, int64_t ldw, double* out2,
                             float* col_norms, float* row_norms, void* ws, size_t ws_bytes,
                             void* stream) {
  if (!W || !out2) return fail(KRONQ_EINVAL, "kronq_weight_cv: NULL pointer");
  if (m < 1 || n < 1 || ldw < n) return fail(KRONQ_EINVAL, "kronq_weight_cv: bad shape");
  size_t need = cv_ws_bytes(m, n);
  const kronq_status st = check_ws("kronq_weight_cv", ws, ws_bytes, need, true);
  if (st) return st;
  return cv_launch(W, m, n, ldw, out2, col_norms, row_norms, ws, (hipStream_t)stream);
}

int64_t kronq_packed_row_bytes(int64_t n, int32_t bits) {
  if (n < 1 || bits < 1 || bits > 8) return 0;
  return decode_row_bytes(n, bits);
}

kronq_status kronq_pack_codes(const uint8_t* codes, int64_t m, int64_t n, int64_t ldc,
                              int32_t bits, const int32_t* perm, uint8_t* packed, int64_t ldp,
                              void* stream) {
  if (!codes || !packed) return fail(KRONQ_EINVAL, "kronq_pack_codes: NULL pointer");
  if (bits != 2 && bits != 4)
    return fail(KRONQ_EINVAL, "kronq_pack_codes: bits %d (only 2 and 4 are packed)", (int)bits);
  if (m < 1 || n < 1 || ldc < n || ldp < decode_row_bytes(n, bits))
    return fail(KRONQ_EINVAL, "kronq_pack_codes: bad shape");
  return pack_launch(codes, m, n, ldc, bits, perm, packed, ldp, (hipStream_t)stream);
}

kronq_status kronq_unpack_codes(const uint8_t* packed, int64_t m, int64_t n, int64_t ldp,
                                int32_t bits, uint8_t* codes, int64_t ldc, void* stream) {
  if (!codes || !packed) return fail(KRONQ_EINVAL, "kronq_unpack_codes: NULL pointer");
  if (bits != 2 && bits != 4)
    return fail(KRONQ_EINVAL, "kronq_unpack_codes: bits %d (only 2 and 4 are packed)", (int)bits);
  if (m < 1 || n < 1 || ldc < n || ldp < decode_row_bytes(n, bits))
    return fail(KRONQ_EINVAL, "kronq_unpack_codes: bad shape");
  return unpack_launch(packed, m, n, ldp, bits, codes, ldc, (hipStream_t)stream);
}

size_t kronq_decode_ws(int64_t m, int64_t n, int32_t bits) {
  if (m < 1 || n < 1 || bits < 1 || bits > 8) return 0;
  return decode_ws_bytes(m, n, bits);
}

kronq_status kronq_decode_matvec(const uint8_t* codes, int64_t m, int64_t n, int64_t ldp,
                                 const kronq_qcfg* q, const float* scales, const float* zeros,
                                 const int32_t* perm, const kronq_had* in_side,
                                 const kronq_had* out_side, const float* sg, const float* x,
                                 float* y, void* ws, size_t ws_bytes, void* stream) {
  kronq_status st = check_decode("kronq_decode_matvec", codes, m, n, ldp, q, scales, zeros, perm,
                                 in_side, out_side, x, y);
  if (st) return st;
  size_t need = decode_ws_bytes(m, n, q->bits);
  st = check_ws("kronq_decode_matvec", ws, ws_bytes, need, true);
  if (st) return st;
  return decode_launch(codes, m, n, ldp, q->bits, q->group > 0 ? q->group : 0, scales, zeros,
                       perm, *in_side, *out_side, sg, x, y, ws, (hipStream_t)stream);
}

kronq_status kronq_decode_matvec_noalloc(const uint8_t* codes, int64_t m, int64_t n, int64_t ldp,
                                         const kronq_qcfg* q, const float* scales,
                                         const float* zeros, const int32_t* perm,
                                         const kronq_had* in_side, const kronq_had* out_side,
                                         const float* sg, const float* x, float* y, void* stream) {
  kronq_status st = check_decode("kronq_decode_matvec_noalloc", codes, m, n, ldp, q, scales, zeros,
                                 perm, in_side, out_side, x, y);
  if (st) return st;
  return decode_launch_noalloc(codes, m, n, ldp, q->bits, q->group > 0 ? q->group : 0, scales, zeros,
                               perm, *in_side, *out_side, sg, x, y, (hipStream_t)stream);
}

size_t kronq_decode_noalloc_max_bytes(void) { return decode_scratch_bytes(); }

kronq_status kronq_sensitivity(const float* HX, int64_t n, int64_t ldhx, const float* HG,
                               int64_t m, int64_t ldhg, double* out3, void* stream) {
  if (!HX || !HG || !out3) return fail(KRONQ_EINVAL, "kronq_sensitivity: NULL pointer");
  if (n < 1 || m < 1 || ldhx < n || ldhg < m)
    return fail(KRONQ_EINVAL, "kronq_sensitivity: bad shape");
  return trace_launch(HX, n, ldhx, HG, m, ldhg, out3, (hipStream_t)stream);
}

}  // extern "C"

namespace {

// Shared checks of the allocators; on success `total` = sum(n_params).
kronq_status alloc_check(const char* fn, int32_t L, const double* scores, const int64_t* n_params,
                         int32_t bmin, int32_t bmax, int64_t budget_bits, int32_t* bits_out,
                         __int128& total) {
  if (L < 1 || !scores || !n_params || !bits_out)
    return fail(KRONQ_EINVAL, "%s: bad arguments", fn);
  if (bmin < 1 || bmax < bmin || bmax > 64)
    return fail(KRONQ_EINVAL, "%s: bad bit range [%d, %d]", fn, (int)bmin, (int)bmax);
  total = 0;
  for (int32_t i = 0; i < L; ++i) {
    if (n_params[i] < 1) return fail(KRONQ_EINVAL, "%s: n_params[%d] < 1", fn, (int)i);
    if (std::isnan(scores[i])) return fail(KRONQ_EINVAL, "%s: score %d is NaN", fn, (int)i);
    total += (__int128)n_params[i];
  }
  if ((__int128)budget_bits < total * bmin)
    return fail(KRONQ_EINVAL, "%s: budget below bmin for every sublayer", fn);
  return KRONQ_OK;
}

// sublayers by descending score, ties to the lower index
std::vector<int32_t> score_order(int32_t L, const double* scores) {
  std::vector<int32_t> order((size_t)L);
  for (int32_t i = 0; i < L; ++i) order[(size_t)i] = i;
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t a, int32_t b) { return scores[a] > scores[b]; });
  return order;
}

}  // namespace

extern "C" {

kronq_status kronq_allocate_bits(int32_t L, const double* scores, const int64_t* n_params,
                                 int32_t bmin, int32_t bmax, int64_t budget_bits,
                                 int32_t* bits_out) {
  __int128 total;
  kronq_status st = alloc_check("kronq_allocate_bits", L, scores, n_params, bmin, bmax,
                                budget_bits, bits_out, total);
  if (st) return st;
  __int128 used = total * bmin;
  for (int32_t i = 0; i < L; ++i) bits_out[i] = bmin;
  for (int32_t i : score_order(L, scores)) {
    while (bits_out[i] < bmax && used + (__int128)n_params[i] <= (__int128)budget_bits) {
      bits_out[i] += 1;
      used += n_params[i];
    }
  }
  return KRONQ_OK;
}

kronq_status kronq_allocate_bits_passwise(int32_t L, const double* scores,
                                          const int64_t* n_params, int32_t bmin, int32_t bmax,
                                          int64_t budget_bits, int32_t* bits_out) {
  __int128 total;
  kronq_status st = alloc_check("kronq_allocate_bits_passwise", L, scores, n_params, bmin, bmax,
                                budget_bits, bits_out, total);
  if (st) return st;
  __int128 used = total * bmin;
  for (int32_t i = 0; i < L; ++i) bits_out[i] = bmin;
  const std::vector<int32_t> order = score_order(L, scores);
  for (bool changed = true; changed;) {
    changed = false;
    for (int32_t i : order)
      if (bits_out[i] < bmax && used + (__int128)n_params[i] <= (__int128)budget_bits) {
        bits_out[i] += 1;
        used += n_params[i];
        changed = true;
      }
  }
  return KRONQ_OK;
}

kronq_status kronq_allocate_bits_marginal(int32_t L, const double* scores,
                                          const int64_t* n_params, int32_t bmin, int32_t bmax,
                                          int64_t budget_bits, int32_t* bits_out) {
  __int128 total;
  kronq_status st = alloc_check("kronq_allocate_bits_marginal", L, scores, n_params, bmin, bmax,
                                budget_bits, bits_out, total);
  if (st) return st;
  __int128 used = total * bmin;
  for (int32_t i = 0; i < L; ++i) bits_out[i] = bmin;
  // loss reduction per bit of one more bit: s 4^-b / n (ldexp is exact, one rounding in the divide)
  auto gain = [&](int32_t i) { return std::ldexp(scores[i], -2 * bits_out[i]) / (double)n_params[i]; };
  for (;;) {
    int32_t best = -1;
    double gbest = 0.0;
    for (int32_t i = 0; i < L; ++i) {
      if (bits_out[i] >= bmax || used + (__int128)n_params[i] > (__int128)budget_bits) continue;
      const double gi = gain(i);
      if (best < 0 || gi > gbest) {
        best = i;
        gbest = gi;
      }
    }
    if (best < 0) return KRONQ_OK;
    bits_out[best] += 1;
    used += n_params[best];
  }
}

kronq_status kronq_allocate_types(int32_t L, const double* scores, const int32_t* type_of,
                                  int32_t n_types, int32_t base_bits, int32_t n_upgrade,
                                  int32_t* bits_out) {
  if (L < 1 || !scores || !type_of || !bits_out || n_types < 1)
    return fail(KRONQ_EINVAL, "kronq_allocate_types: bad arguments");
  if (base_bits < 1 || base_bits > 63 || n_upgrade < 0 || n_upgrade > n_types)
    return fail(KRONQ_EINVAL, "kronq_allocate_types: base_bits %d / n_upgrade %d out of range",
                (int)base_bits, (int)n_upgrade);
  std::vector<double> sum((size_t)n_types, 0.0);
  for (int32_t i = 0; i < L; ++i) {
    if (type_of[i] < 0 || type_of[i] >= n_types)
      return fail(KRONQ_EINVAL, "kronq_allocate_types: type_of[%d] = %d outside [0, %d)", (int)i,
                  (int)type_of[i], (int)n_types);
    if (std::isnan(scores[i])) return fail(KRONQ_EINVAL, "kronq_allocate_types: score %d is NaN", (int)i);
    sum[(size_t)type_of[i]] += scores[i];   // ascending sublayer order
  }
  const std::vector<int32_t> ranked = score_order(n_types, sum.data());
  std::vector<char> up((size_t)n_types, 0);
  for (int32_t k = 0; k < n_upgrade; ++k) up[(size_t)ranked[(size_t)k]] = 1;
  for (int32_t i = 0; i < L; ++i) bits_out[i] = base_bits + (up[(size_t)type_of[i]] ? 1 : 0);
  return KRONQ_OK;
}

}  // extern "C"
