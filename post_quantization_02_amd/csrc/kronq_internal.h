// Internal declarations shared by the host API and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "kronq.h"

namespace kronq {

// Thread-local error detail behind kronq_last_error().
void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
kronq_status fail(kronq_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
kronq_status hip_fail(hipError_t e, const char* what);

#define KQ_HIP(call)                                              \
  do {                                                            \
    hipError_t _e = (call);                                       \
    if (_e != hipSuccess) return ::kronq::hip_fail(_e, #call);    \
  } while (0)

#define KQ_LAUNCHED(name)                                         \
  do {                                                            \
    hipError_t _e = hipGetLastError();                            \
    if (_e != hipSuccess) return ::kronq::hip_fail(_e, name);     \
  } while (0)

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---- launchers (one translation unit per kernel family) ----

// gram.hip
size_t gram_ws_bytes(int64_t N, int64_t d, int32_t dtype);
kronq_status gram_launch(const void* A, int32_t dtype, int64_t N, int64_t d, int64_t lda, float* H,
                         int64_t ldh, float scale, float beta, void* ws, size_t ws_bytes,
                         hipStream_t s);

// whether the direct-to-LDS Gram pipeline can address an operand with this
// leading dimension (32-bit offsets within a stage)
bool gram_pipeline_ld_ok(int64_t ld);
size_t gram_cross_ws_bytes(int64_t N, int64_t d);
kronq_status gram_cross_launch(const void* A, const void* B, int64_t N, int64_t d, int64_t ld, float* C,
                               int64_t ldc, float scale, float beta, const float* sub, int64_t ldsub,
                               void* ws, hipStream_t s);

// fwht.hip
size_t biip_ws_bytes(int64_t m, int64_t n);
// rescale_in: also the input-side rescale (sx_in when given, else diag(HX)^alpha_x;
// written to sx_out when computed); W may then be NULL.  Workspace biip_sx_ws_bytes.
kronq_status biip_launch(float* W, int64_t m, int64_t n, int64_t ldw, float* HX, int64_t ldhx,
                         float* HG, int64_t ldhg, const kronq_had& in, const kronq_had& out,
                         float alpha, float* sg, void* ws, size_t ws_bytes, hipStream_t s,
                         bool rescale_in = false, float alpha_x = 0.0f,
                         const float* sx_in = nullptr, float* sx_out = nullptr);
size_t biip_sx_ws_bytes(int64_t m, int64_t n);

size_t unrotate_ws_bytes(int64_t m);
kronq_status unrotate_launch(float* W, int64_t m, int64_t n, int64_t ldw, const kronq_had& in,
                             const kronq_had& out, const float* sg, void* ws, hipStream_t s);
size_t unrotate_sx_ws_bytes(int64_t m, int64_t n);
kronq_status unrotate_sx_launch(float* W, int64_t m, int64_t n, int64_t ldw, const kronq_had& in,
                                const kronq_had& out, const float* sg, const float* sx, void* ws,
                                hipStream_t s);

// chol.hip
size_t chol_ws_bytes(int64_t n);
kronq_status chol_launch(const float* H, int64_t n, int64_t ldh, float lambda, int act_order,
                         int32_t* perm, float* R, int64_t ldr, int64_t* info, void* ws,
                         size_t ws_bytes, hipStream_t s);

// gptq.hip
size_t gptq_ws_bytes(int64_t m, int64_t n);
kronq_status gptq_launch(const float* W, int64_t m, int64_t n, int64_t ldw, const float* R,
                         int64_t ldr, const int32_t* perm, int bits, int group, uint8_t* codes,
                         float* scales, float* zeros, float* What, float* pre_round,
                         double* row_loss, void* ws, size_t ws_bytes, hipStream_t s,
                         const float* Wp = nullptr, const float* X2 = nullptr);

// gptaq.hip
size_t gptaq_correction_ws_bytes(int64_t n);
kronq_status gptaq_correction_launch(const float* C, int64_t n, int64_t ldc, const float* R, int64_t ldr,
                                     const int32_t* perm, float alpha, float* P, int64_t ldp, void* ws,
                                     hipStream_t s);
size_t drift_cross_ws_bytes(int64_t N, int64_t n);
kronq_status drift_cross_launch(const void* Xfp, const void* X, int64_t N, int64_t n, int64_t ld, float* C,
                                int64_t ldc, void* ws, hipStream_t s);
size_t gptaq_shift_ws_bytes(int64_t m, int64_t n);
kronq_status gptaq_shift_launch(const float* W, int64_t m, int64_t n, int64_t ldw, const int32_t* perm,
                                const float* P, int64_t ldp, int unit, float* W1, float* X2,
                                hipStream_t s);

// trace.hip
kronq_status trace_launch(const float* HX, int64_t n, int64_t ldhx, const float* HG, int64_t m,
                          int64_t ldhg, double* out3, hipStream_t s);

// diag.hip
size_t cv_ws_bytes(int64_t m, int64_t n);
kronq_status finite_launch(const float* A, int64_t rows, int64_t cols, int64_t ld, int32_t* flag,
                           hipStream_t s);
kronq_status cv_launch(const float* W, int64_t m, int64_t n, int64_t ldw, double* out2,
                       float* col_norms, float* row_norms, void* ws, hipStream_t s);

// eig.hip
size_t eig_ws_bytes(int64_t n);
kronq_status eig_launch(const float* H, int64_t n, int64_t ldh, double tol, int max_sweeps,
                        double* mu, double* evals, double* Q, int64_t ldq, int32_t* sweeps, void* ws,
                        hipStream_t s);

// codec.hip
kronq_status pack_launch(const uint8_t* codes, int64_t m, int64_t n, int64_t ldc, int bits,
                         const int32_t* perm, uint8_t* packed, int64_t ldp, hipStream_t s);
kronq_status unpack_launch(const uint8_t* packed, int64_t m, int64_t n, int64_t ldp, int bits,
                           uint8_t* codes, int64_t ldc, hipStream_t s);
int64_t decode_row_bytes(int64_t n, int bits);
size_t decode_ws_bytes(int64_t m, int64_t n, int bits);
kronq_status decode_launch(const uint8_t* codes, int64_t m, int64_t n, int64_t ldp, int bits,
                           int64_t group, const float* scales, const float* zeros,
                           const int32_t* perm, const kronq_had& in, const kronq_had& out,
                           const float* sg, const float* x, float* y, void* ws, hipStream_t s);
size_t decode_scratch_bytes();
kronq_status decode_launch_noalloc(const uint8_t* codes, int64_t m, int64_t n, int64_t ldp, int bits,
                                   int64_t group, const float* scales, const float* zeros,
                                   const int32_t* perm, const kronq_had& in, const kronq_had& out,
                                   const float* sg, const float* x, float* y, hipStream_t s);

}  // namespace kronq
