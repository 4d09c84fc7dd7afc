/*
 * kronq.h -- C ABI of the KronQ per-sublayer quantization path on AMD Instinct
 * MI355X (gfx950).
 *
 * The method (KronQ, arXiv 2607.07964, "KronQ: LLM Quantization via
 * Kronecker-Factored Hessian"; pages cited below by name and section):
 *   1. Kronecker factors H_X = X^T X / N and H_G = G^T G / N of the K-FAC
 *      Hessian H ~ H_X (x) H_G            (hyper.ai summary, Method)
 *   2. bidirectional incoherence processing: output rescale S_G and randomized
 *      Hadamard transforms on both sides  (hyper.ai summary, Method; Pith
 *      review, Eq. 11-12 and the proof of Theorem 1)
 *   3. damping and the inverse Cholesky factor of H_X (Pith review, Algorithm 2)
 *   4. the column-wise OBS quantize-and-compensate loop with H_X alone, since
 *      H_G cancels                       (Pith review, Proposition 1)
 *   5. the sensitivity tr(H_X) tr(H_G) and the bit allocation it drives
 *                                         (hyper.ai summary, Method, Eq. 14)
 *
 * Conventions for every call:
 *   - All matrices are row-major; leading dimensions are in elements.
 *   - Device pointers are HIP device memory owned by the caller; the library
 *     never allocates, frees or retains caller memory.  Calls that need scratch
 *     memory take a caller-provided device workspace `ws` of at least the size
 *     returned by the matching *_ws() query (KRONQ_EWORKSPACE otherwise),
 *     16-byte aligned (KRONQ_EINVAL otherwise; any hipMalloc or torch
 *     allocation is).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Device calls are
 *     asynchronous on `stream` except kronq_chol_inv, which synchronizes it.
 *   - Arguments are validated on the host before anything is launched; an
 *     invalid argument returns KRONQ_EINVAL and launches nothing.  HIP runtime
 *     failures return KRONQ_EHIP.  kronq_last_error() gives a readable detail
 *     of the last failure on the calling thread.
 *   - The library keeps no state between calls: calls on different streams may
 *     run concurrently as long as their buffers do not overlap.
 */
#ifndef KRONQ_H
#define KRONQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t kronq_status;
#define KRONQ_OK 0
#define KRONQ_EINVAL 1         /* invalid argument (nothing launched) */
#define KRONQ_ENOTPD 2         /* damped H not positive definite */
#define KRONQ_EHIP 3           /* HIP runtime error */
#define KRONQ_EWORKSPACE 4     /* workspace smaller than the *_ws() size */
#define KRONQ_EUNSUPPORTED 5   /* valid request the library does not implement */
#define KRONQ_ENUMERIC 6       /* input holds a NaN or an infinity (found on the device) */
#define KRONQ_ENOMEM 7         /* request larger than a fixed device buffer of the library */

#define KRONQ_F32 0            /* element type codes for kronq_gram */
#define KRONQ_BF16 1

/* One side of a randomized (block) Hadamard transform T = (I_b (x) H_block)
 * diag(signs) / sqrt(block) on a dimension dim = b * block; block is a power of
 * two (Sylvester order) between 1 and 32768; signs is a device array of dim
 * floats, each +1.0f or -1.0f (the random draw is the caller's input).
 * block = 1 with signs = NULL is the identity: a side left unprocessed, as in
 * the incoherence ablations (GitHub README, --incoh_mode su_only / sv_only). */
typedef struct {
  int64_t dim;
  int64_t block;
  const float* signs;
} kronq_had;

/* Quantizer of the column loop: asymmetric uniform grid with 2^bits levels
 * (bits in 1..8); group <= 0 means one grid per output row (per-channel),
 * otherwise one grid per `group` consecutive columns in processing order
 * (group must divide n). */
typedef struct {
  int32_t bits;
  int32_t group;
} kronq_qcfg;

const char* kronq_status_string(kronq_status s);
const char* kronq_last_error(void);
int32_t kronq_version(void);

/* ---------------------------------------------------------------------------
 * Random signs of the randomized Hadamard transforms (hyper.ai summary, Method:
 * U and V are randomized Hadamard transforms; GitHub README: the incoherence
 * machinery follows QuIP#, whose randomized Hadamard transform multiplies by
 * random signs before the transform).  The pages fix no generator; this is
 * the library's documented draw, so that a caller can reproduce a rotation
 * from its seed alone.  With the public splitmix64 finalizer
 *   mix(z): z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9;
 *           z = (z ^ (z >> 27)) * 0x94D049BB133111EB; return z ^ (z >> 31)
 * (Steele, Lea and Flood, OOPSLA 2014) and its increment g = 0x9E3779B97F4A7C15:
 *   key   = mix(mix(seed) ^ (6 * g))
 *   out[i] = top bit of mix(key + (i + 1) * g) ? -1.0f : +1.0f,  i = 0..n-1
 * (all products modulo 2^64).  out_host: host array of n floats.  KRONQ_EINVAL
 * for n < 0 or out_host NULL with n > 0.  Host only; thread safe.
 * ------------------------------------------------------------------------- */
kronq_status kronq_signs(uint64_t seed, int64_t n, float* out_host);

/* ---------------------------------------------------------------------------
 * Finiteness check of a device matrix (the library's guard against NaN and
 * infinite values: kronq_chol_inv applies it to its input and returns
 * KRONQ_ENUMERIC; the asynchronous calls cannot report a device-side finding
 * as a status, so a caller checks their inputs or outputs with this call).
 *   flag_dev (device int32) <- 1 if some A[i][j], i < rows, j < cols, is NaN or
 *                              infinite, else 0
 * A : rows x cols fp32 device, leading dimension ld >= cols (read only).
 * Two launches on `stream` (clear, then scan), no host synchronization and no
 * memset; the caller reads flag_dev after synchronizing.  rows or cols 0
 * writes 0.
 * ------------------------------------------------------------------------- */
kronq_status kronq_check_finite(const float* A, int64_t rows, int64_t cols, int64_t ld,
                                int32_t* flag_dev, void* stream);

/* ---------------------------------------------------------------------------
 * Kronecker factor (hyper.ai summary, Method: H_X = E[x x^T], H_G = E[g g^T]
 * under the K-FAC factorization).
 *   H <- scale * A^T A + beta * H
 * A     : N x d device matrix, row-major with leading dimension lda >= d, of
 *         element type dtype (KRONQ_BF16 or KRONQ_F32); one token per row.
 * H     : d x d device fp32, leading dimension ldh >= d; both triangles are
 *         written (full symmetric storage).  With beta == 0, H is not read.
 * scale : typically 1/N; beta = 1 accumulates token chunks.
 * bf16 products are exact in fp32 and accumulate in fp32 on the bf16 matrix
 * cores; fp32 input uses the fp32 matrix cores.
 * ws    : device workspace of kronq_gram_ws(N, d, dtype) bytes (may be 0).
 * Requires N >= 1, d >= 1, A and H 16-byte aligned, lda a multiple of 8
 * (bf16) or 4 (f32).
 * ------------------------------------------------------------------------- */
size_t kronq_gram_ws(int64_t N, int64_t d, int32_t dtype);
kronq_status kronq_gram(const void* A, int32_t dtype, int64_t N, int64_t d, int64_t lda, float* H,
                        int64_t ldh, float scale, float beta, void* ws, size_t ws_bytes,
                        void* stream);

/* ---------------------------------------------------------------------------
 * Bidirectional incoherence processing (hyper.ai summary, Method: rescale on
 * the output side by S_G, then orthogonal transforms; Pith review, proof of
 * Theorem 1: W' = U W V^T, H_G' = U H_G U^T, H_X' = V H_X V^T).
 *   sg[i] = HG[i][i]^alpha  (1 where HG[i][i] <= 0; all 1 when alpha == 0)
 *   W  (m x n) <- U diag(sg) W V^T
 *   HX (n x n) <- V HX V^T
 *   HG (m x m) <- U diag(sg)^-1 HG diag(sg)^-1 U^T
 * with U from out_side (dim m) and V from in_side (dim n), in place, fp32.
 * HX may be NULL (skipped, e.g. when sublayers share an already rotated H_X);
 * HG may be NULL only when alpha == 0 (then sg is all ones).  sg (device,
 * m floats) may be NULL.  W and HX/HG must not overlap.
 * ws : kronq_biip_ws(m, n) bytes.
 * ------------------------------------------------------------------------- */
size_t kronq_biip_ws(int64_t m, int64_t n);
kronq_status kronq_biip_rotate(float* W, int64_t m, int64_t n, int64_t ldw, float* HX,
                               int64_t ldhx, float* HG, int64_t ldhg, const kronq_had* in_side,
                               const kronq_had* out_side, float alpha, float* sg, void* ws,
                               size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Inverse of the weight side of BiIP, back to the original domain (Pith
 * review, Theorem 1: U and V are orthogonal, so W = U^T W' V; hyper.ai summary,
 * Method: the S_G rescale was applied first and is divided out last).
 *   W (m x n) <- diag(sg)^-1 U^T W V      in place, fp32
 * with U from out_side (dim m) and V from in_side (dim n), the same specs and
 * sg that kronq_biip_rotate was given (sg NULL: no rescale).  Applied to the
 * dequantized W'^ it gives the quantized layer in its original basis.
 * ws : kronq_biip_unrotate_ws(m, n) bytes.
 * ------------------------------------------------------------------------- */
size_t kronq_biip_unrotate_ws(int64_t m, int64_t n);
kronq_status kronq_biip_unrotate(float* W, int64_t m, int64_t n, int64_t ldw,
                                 const kronq_had* in_side, const kronq_had* out_side,
                                 const float* sg, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * BiIP with the input-side rescale S_X as well (hyper.ai summary, Method: the
 * input-side diagonal rescaling is extended to both directions, S_G being the
 * output-side part; Pith review, Algorithm 1 returns S_X beside S_G, U, V).
 * The input side takes the form of the output side:
 *   sx[j] = HX[j][j]^alpha_x  (1 where HX[j][j] <= 0; all 1 when alpha_x == 0),
 *           read from H_X before it is transformed
 *   W  (m x n) <- U diag(sg) W diag(sx) V^T
 *   HX (n x n) <- V diag(sx)^-1 HX diag(sx)^-1 V^T
 *   HG (m x m) <- as kronq_biip_rotate
 * which keeps the proxy loss tr(H_G dW H_X dW^T) of a perturbation dW that is
 * transformed as W is.  Arguments as kronq_biip_rotate, plus:
 *   alpha_x  : exponent of the input rescale.
 *   sx       : device, n floats.  sx_given = 0: the computed rescale is written
 *              there (sx may be NULL); HX is required unless alpha_x == 0.
 *              sx_given = 1: sx is read (nonzero finite values, e.g. from an
 *              earlier call on the same input) and alpha_x is ignored; HX may
 *              then be NULL (a shared H_X already transformed) or any n x n
 *              matrix that transforms as H_X does -- the drift cross product
 *              of kronq_drift_cross, with W and HG NULL.
 *   W may be NULL (only HX and HG are transformed); not all of W, HX, HG NULL.
 * The deploy decode of a layer rescaled this way takes x' = V diag(sx)^-1 x:
 * kronq_decode_matvec multiplies by its input-side signs array, so a caller
 * passes the product D_in[j] / sx[j] there.
 * ws : kronq_biip_sx_ws(m, n) bytes (required).
 * ------------------------------------------------------------------------- */
size_t kronq_biip_sx_ws(int64_t m, int64_t n);
kronq_status kronq_biip_rotate_sx(float* W, int64_t m, int64_t n, int64_t ldw, float* HX,
                                  int64_t ldhx, float* HG, int64_t ldhg, const kronq_had* in_side,
                                  const kronq_had* out_side, float alpha, float alpha_x, float* sg,
                                  float* sx, int32_t sx_given, void* ws, size_t ws_bytes,
                                  void* stream);

/* Inverse of the weight side of kronq_biip_rotate_sx:
 *   W (m x n) <- diag(sg)^-1 U^T W V diag(sx)^-1      in place, fp32
 * sx (device, n floats) as returned by kronq_biip_rotate_sx; sg as in
 * kronq_biip_unrotate.  ws : kronq_biip_unrotate_sx_ws(m, n) bytes. */
size_t kronq_biip_unrotate_sx_ws(int64_t m, int64_t n);
kronq_status kronq_biip_unrotate_sx(float* W, int64_t m, int64_t n, int64_t ldw,
                                    const kronq_had* in_side, const kronq_had* out_side,
                                    const float* sg, const float* sx, void* ws, size_t ws_bytes,
                                    void* stream);

/* ---------------------------------------------------------------------------
 * Act-order, damping and inverse Cholesky factor (Pith review, Algorithm 2:
 * the damped H_X is H_X + lambda mean(diag H_X) I and the loop uses its
 * inverse Cholesky factor; GitHub README, flag --act_order).
 *   perm  : if act_order, the stable descending order of diag(H) (ties to the
 *           lower index); else the identity.  perm[j] = original column
 *           processed at step j.  Device int32[n].
 *   Hd    = P (H + lambda * mean(diag H) * I) P^T
 *   R     : upper triangular, positive diagonal, R^T R = Hd^-1 (fp32, lower
 *           triangle written as zeros).  Device, leading dimension ldr.
 * H is read only (n x n fp32 device, symmetric).  Computed in fp32 on the
 * matrix cores (blocked factorization of the reversed matrix, then a blocked
 * triangular inverse).
 * info  : host pointer; -1 on success.  When Hd is not positive definite,
 *         KRONQ_ENOTPD is returned and info is the largest k (processing
 *         order) whose trailing block Hd[k:, k:] is not positive definite
 *         (the factorization runs on the reversed matrix, so this is where its
 *         first non-positive pivot falls).  When H holds a NaN or an
 *         infinity (or its damping term is not finite), KRONQ_ENUMERIC is
 *         returned instead, info stays -1 and R is not written.
 * All work runs on `stream`, which is synchronized before returning (the
 * flag of a failed pivot is read back).
 * ws    : kronq_chol_inv_ws(n) bytes.
 * ------------------------------------------------------------------------- */
size_t kronq_chol_inv_ws(int64_t n);
kronq_status kronq_chol_inv(const float* H, int64_t n, int64_t ldh, float lambda,
                            int32_t act_order, int32_t* perm, float* R, int64_t ldr,
                            int64_t* info, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Column-wise OBS quantize-and-compensate with H_X alone (Pith review,
 * Proposition 1: H_G cancels from the column update; Algorithm 2: lazy
 * batches of columns).  For every row independently and for j = 0..n-1 in
 * processing order (column c = perm[j]):
 *   t = w[c] / scale + zero;  q = clamp(round-half-even(t), 0, 2^bits - 1)
 *   wq = scale * (q - zero);  e = (w[c] - wq) / R[j][j]
 *   w[perm[k]] -= e * R[j][k]   for k > j
 * Grid parameters: xmin = min(0, min v), xmax = max(0, max v) (a degenerate
 * range becomes [-1, 1]), scale = (xmax - xmin) / (2^bits - 1),
 * zero = round-half-even(-xmin / scale), with v the whole initial row
 * (per-channel) or the current compensated values of the group when its first
 * column is reached.  The loop runs in fp64 (inputs fp32).
 * W        : m x n fp32 device, natural column order (read only).
 * R        : n x n fp32 device upper factor in processing order, 16-byte
 *            aligned with ldr a multiple of 4 (else KRONQ_EINVAL).
 * perm     : device int32[n] or NULL (identity).
 * codes    : m x n uint8 device, natural column order, leading dimension n.
 * scales, zeros : m x ngroups fp32 device (ngroups = 1 per-channel, else
 *            n / group), groups in processing order, leading dimension ngroups.
 * What     : m x n fp32 device dequantized weights, natural order, leading
 *            dimension n; may be NULL.  May alias W when ldw == n.
 * pre_round: m x n fp32 device t values (natural order) or NULL.
 * row_loss : m fp64 device values or NULL: row_loss[r] = sum_j e_j^2 over the
 *            row's scaled errors e_j (processing order), summed in fp64.
 *            Since the weight change of the row is e R (R's rows in
 *            processing order), this is the row's proxy loss
 *            (W - What)[r] Hd (W - What)[r]^T with H_G = I (the LDL form of the
 *            GPTQ bound, Pith review, Table 9).
 * Group sizes: group > 0 must also be a multiple of 8 that divides 128
 *            (8, 16, 32, 64, 128): a group's grid comes from the current
 *            values of one 128-column block of the loop.  Other sizes that
 *            divide n return KRONQ_EUNSUPPORTED.
 * ws       : kronq_gptq_ws(m, n) bytes.
 * ------------------------------------------------------------------------- */
size_t kronq_gptq_ws(int64_t m, int64_t n);
kronq_status kronq_gptq_quantize(const float* W, int64_t m, int64_t n, int64_t ldw,
                                 const float* R, int64_t ldr, const int32_t* perm,
                                 const kronq_qcfg* q, uint8_t* codes, float* scales,
                                 float* zeros, float* What, float* pre_round, double* row_loss,
                                 void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * GPTAQ asymmetric correction (hyper.ai summary, Method: building on GPTAQ the
 * objective corrects for input drift by asymmetric calibration -- the
 * quantized layer sees the inputs X of the partly quantized model while its
 * target is the full-precision layer on the full-precision inputs X_fp;
 * Pith review, Algorithm 2: P = alpha (dXX^T L) (.) M_U L^T after the inverse
 * Cholesky step, used by the column loop; proof of Theorem 1:
 * (dXX^T)' = V dXX^T V^T).  The column update that uses P is cut off on the
 * pages; the library's reading is the sequential OBS in which column j's drift
 * is committed once it is quantized: every later column k then also moves by
 * + w_j P[j][k], w_j the full-precision weight of column j, with L = R^T and
 * M_U the strictly upper mask.
 *
 * kronq_drift_cross: the drift term C = (X_fp - X)^T X / N (the pages' dXX^T
 *   in the normalization of H_X), X_fp and X N x n bf16 (same leading
 *   dimension ld, a multiple of 8; 16-byte aligned), C n x n fp32 (ldc).
 *   dX = X_fp - X is formed exactly in fp32 and split into two bf16 parts (hi
 *   + lo, 16 significant bits: exact unless X_fp and X differ by more than a
 *   factor 2^8), then hi^T X + lo^T X accumulates in fp32 on the bf16 matrix
 *   cores, in chunks of 32768 tokens.  n must be a multiple of 256, N of 128
 *   and ld at most 67108848 (KRONQ_EUNSUPPORTED otherwise: the pipeline
 *   addresses a stage with 32-bit offsets).  ws: kronq_drift_cross_ws(N, n)
 *   bytes.  The input side of BiIP applies to C as to H_X: C' = V C V^T is
 *   kronq_biip_rotate with W = C, both sides the input side's spec, HX and HG
 *   NULL and alpha 0.
 * kronq_gram_cross: the general cross product C = scale A^T B - sub (A and B
 *   N x d bf16 with one layout as above, sub d x d fp32 or NULL), on the same
 *   tiles, with the same limits on d, N and ld.  ws: kronq_gram_cross_ws(N, d)
 *   bytes.
 * kronq_gptaq_correction: P = alpha ((C_p R^T) (.) M) R with
 *   C_p[a][b] = C[perm[a]][perm[b]] (perm NULL: identity), R the n x n upper
 *   factor of kronq_chol_inv (processing order, lower triangle zero) and M the
 *   strictly upper mask; P is n x n fp32 (ldp), strictly upper triangular
 *   (zeros written on and below the diagonal).  fp32 on the matrix cores.
 *   ws: kronq_gptaq_correction_ws(n) bytes.
 * kronq_gptaq_quantize: kronq_gptq_quantize with the drift term: as there,
 *   and after column j (processing order) is quantized every later column k
 *   also moves by + W[r][perm[j]] P[j][k] (P n x n fp32, processing order,
 *   strictly upper, ldp).  The drift shifts are formed up front on the fp32
 *   matrix cores; a group's grid includes the drift of every earlier column;
 *   the loop runs in fp64.  row_loss reports the sum of the squared scaled
 *   errors (w~_j - wq_j) / R_jj.  Groups as kronq_gptq_quantize.  What may
 *   alias W when ldw == n.  ws: kronq_gptaq_ws(m, n) bytes.
 * ------------------------------------------------------------------------- */
size_t kronq_drift_cross_ws(int64_t N, int64_t n);
kronq_status kronq_drift_cross(const void* Xfp, const void* X, int64_t N, int64_t n, int64_t ld, float* C,
                               int64_t ldc, void* ws, size_t ws_bytes, void* stream);
size_t kronq_gram_cross_ws(int64_t N, int64_t d);
kronq_status kronq_gram_cross(const void* A, const void* B, int64_t N, int64_t d, int64_t ld, float* C,
                              int64_t ldc, float scale, const float* sub, int64_t ldsub, void* ws,
                              size_t ws_bytes, void* stream);
size_t kronq_gptaq_correction_ws(int64_t n);
kronq_status kronq_gptaq_correction(const float* C, int64_t n, int64_t ldc, const float* R, int64_t ldr,
                                    const int32_t* perm, float alpha, float* P, int64_t ldp, void* ws,
                                    size_t ws_bytes, void* stream);
size_t kronq_gptaq_ws(int64_t m, int64_t n);
kronq_status kronq_gptaq_quantize(const float* W, int64_t m, int64_t n, int64_t ldw, const float* R,
                                  int64_t ldr, const int32_t* perm, const kronq_qcfg* q, const float* P,
                                  int64_t ldp, uint8_t* codes, float* scales, float* zeros, float* What,
                                  float* pre_round, double* row_loss, void* ws, size_t ws_bytes,
                                  void* stream);

/* ---------------------------------------------------------------------------
 * Weight diagnostic of incoherence processing (Pith review, Figure 2: CV_in and
 * CV_out are the coefficients of variation of the column norms and of the row
 * norms of W).
 *   out2[0] = CV_in  = std(||W[:, j]||) / mean(||W[:, j]||)   over the n columns
 *   out2[1] = CV_out = std(||W[i, :]||) / mean(||W[i, :]||)   over the m rows
 * with the population standard deviation; norms from fp32 squares summed in
 * fp32 within 64 x 1024 tiles and fp64 across tiles, statistics in fp64.  NaN
 * when every norm is zero.
 * W        : m x n fp32 device, leading dimension ldw >= n (read only).
 * out2     : device, 2 doubles.
 * col_norms, row_norms : device n and m floats receiving the norms, or NULL.
 * ws       : kronq_weight_cv_ws(m, n) bytes.
 * ------------------------------------------------------------------------- */
size_t kronq_weight_cv_ws(int64_t m, int64_t n);
kronq_status kronq_weight_cv(const float* W, int64_t m, int64_t n, int64_t ldw, double* out2,
                             float* col_norms, float* row_norms, void* ws, size_t ws_bytes,
                             void* stream);

/* ---------------------------------------------------------------------------
 * mu-incoherence of a symmetric matrix (hyper.ai summary, Method, and Pith
 * review, Figure 2(a): mu(H)/sqrt(d) near 1 when an eigenvector lies along a
 * coordinate axis, small once the transforms have spread them out).  With
 * H = Q Lambda Q^T (Q orthogonal):
 *   mu (host double) <- max_ij |Q_ij|       (= mu(H) / sqrt(n))
 * H     : n x n fp32 device, leading dimension ldh >= n; only the lower
 *         triangle is read (the matrix is taken as symmetric).
 * evals : device double[n] or NULL: the eigenvalues, in the order of Q's
 *         columns (not sorted).
 * Q     : device double n x n (leading dimension ldq >= n) or NULL: the
 *         eigenvectors as columns.
 * sweeps: host int32 or NULL: the Jacobi sweeps taken.
 * Computed in fp64 by two-sided block Jacobi (sweeps over all pairs of
 * 16-index blocks, each 32 x 32 pair subproblem diagonalized in full) until the
 * off-diagonal Frobenius norm is at most tol times the Frobenius norm
 * (tol in [1e-15, 1e-2]; 1e-13 is typical and reaches the eigenvectors to
 * about 1e-13 * ||H|| / gap); KRONQ_ENUMERIC when that takes more than
 * max_sweeps sweeps (1..100) or H holds a NaN or an infinity.  Where
 * eigenvalues repeat, Q and so mu are not unique.  Synchronous on `stream`
 * (the host reads the norm after each sweep).  n <= 32768.
 * ws : kronq_incoherence_ws(n) bytes (about 16 n^2).
 * ------------------------------------------------------------------------- */
size_t kronq_incoherence_ws(int64_t n);
kronq_status kronq_incoherence(const float* H, int64_t n, int64_t ldh, double tol, int32_t max_sweeps,
                               double* mu, double* evals, double* Q, int64_t ldq, int32_t* sweeps,
                               void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Deploy codec (GitHub README of the KronQ release: int4 / int2 weights are
 * stored packed and a fused dequantize + BiIP matvec unpacks them on the fly
 * for single-token decode).
 * Packed layout (bits 2 and 4): code j of a row is stored at bit offset
 * bits * (j mod (8 / bits)) of byte j / (8 / bits) of that row, low bits
 * first; a row holds kronq_packed_row_bytes(n, bits) = ceil(n * bits / 8)
 * bytes (the unused high bits of its last byte are zero).  Other widths are
 * stored one code per byte (kronq_packed_row_bytes = n), as
 * kronq_gptq_quantize writes them.
 *
 * kronq_pack_codes: codes (m x n uint8 device, leading dimension ldc >= n) ->
 *   packed (m rows of ldp >= row bytes, device); only the low `bits` bits of a
 *   code are stored; bytes of a row past its row bytes are not written.
 *   perm (device int32[n] or NULL): when given, stored column j holds code
 *   column perm[j], i.e. the codes are stored in the column loop's processing
 *   order, where its groups are contiguous (act-order layers).
 * kronq_unpack_codes: the inverse (codes < 2^bits).
 * Both take bits 2 or 4 (KRONQ_EINVAL otherwise); buffers must not overlap.
 * ------------------------------------------------------------------------- */
int64_t kronq_packed_row_bytes(int64_t n, int32_t bits);
kronq_status kronq_pack_codes(const uint8_t* codes, int64_t m, int64_t n, int64_t ldc,
                              int32_t bits, const int32_t* perm, uint8_t* packed, int64_t ldp,
                              void* stream);
kronq_status kronq_unpack_codes(const uint8_t* packed, int64_t m, int64_t n, int64_t ldp,
                                int32_t bits, uint8_t* codes, int64_t ldc, void* stream);

/* ---------------------------------------------------------------------------
 * Batch-1 decode matvec of a quantized, incoherence-processed layer (GitHub
 * README: fused dequant + BiIP matvec; Pith review, Theorem 1; hyper.ai summary,
 * Method).  With W'^[r][c] = scales[r][g] (q[r][c] - zeros[r][g]):
 *   y = diag(sg)^-1 U^T W'^ V x      computed as  x' = V x,  y' = W'^ x',
 *                                                 y = diag(sg)^-1 U^T y'
 * codes  : m rows of ldp bytes (device, 16-byte aligned, ldp a multiple of 16
 *          and >= kronq_packed_row_bytes(n, q->bits)); packed as above for
 *          bits 2 and 4, one code per byte otherwise.  The whole m x ldp
 *          buffer must be readable (the pad bytes of a row may be read, never
 *          used).
 * q      : bits 1..8; group <= 0 (one grid per row) or a multiple of 64 that
 *          divides n (KRONQ_EUNSUPPORTED for other group sizes); group g covers
 *          stored columns [g * group, (g + 1) * group).
 * scales, zeros : m x ngroups fp32 device, leading dimension ngroups, as
 *          kronq_gptq_quantize writes them (groups in processing order).
 * perm   : NULL when the codes are stored in natural column order (a layer
 *          quantized without act-order, or one grid per row); else the
 *          act-order permutation, device int32[n], with the codes stored in
 *          processing order (stored column j = natural column perm[j], as
 *          kronq_pack_codes writes them when given perm).  Then n <= 32768
 *          (KRONQ_EUNSUPPORTED above): each workgroup builds the whole x'.
 * in_side, out_side, sg : the transforms and rescale of kronq_biip_rotate
 *          (sg device m floats, NULL for no rescale).
 * x      : n fp32 device;  y : m fp32 device (must not overlap x or ws).
 * Arithmetic is fp32.  Two kernel launches on `stream`, no host
 * synchronization and no memset: the call may be captured in a HIP graph
 * (for blocks above 8192 the first call should be made outside capture, since
 * it raises a kernel's LDS limit).
 * ws     : kronq_decode_ws(m, n, bits) bytes.
 * ------------------------------------------------------------------------- */
size_t kronq_decode_ws(int64_t m, int64_t n, int32_t bits);
kronq_status kronq_decode_matvec(const uint8_t* codes, int64_t m, int64_t n, int64_t ldp,
                                 const kronq_qcfg* q, const float* scales, const float* zeros,
                                 const int32_t* perm, const kronq_had* in_side,
                                 const kronq_had* out_side, const float* sg, const float* x,
                                 float* y, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * The same decode for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Arguments, layouts, results and errors are those of kronq_decode_matvec,
 * without the workspace: the per-slice partial sums go to a fixed device
 * buffer inside the library of kronq_decode_noalloc_max_bytes() bytes (4 MiB)
 * per GPU, which each GPU the library runs on holds until the process ends.
 * A request whose partial sums, kronq_decode_ws(m, n, bits), exceed it returns
 * KRONQ_ENOMEM and launches nothing.  The call runs on the calling thread's
 * current device (`stream` must belong to it); its first call on a device
 * looks up the buffer's address once (no allocation).  No hipMalloc, hipFree
 * or allocating library routine is called.  Every call on one GPU shares that
 * GPU's buffer: calls that overlap in time on one GPU (other streams, other
 * threads) race and must be serialized by the caller; calls on one stream are
 * ordered and safe.
 * ------------------------------------------------------------------------- */
size_t kronq_decode_noalloc_max_bytes(void);
kronq_status kronq_decode_matvec_noalloc(const uint8_t* codes, int64_t m, int64_t n, int64_t ldp,
                                         const kronq_qcfg* q, const float* scales,
                                         const float* zeros, const int32_t* perm,
                                         const kronq_had* in_side, const kronq_had* out_side,
                                         const float* sg, const float* x, float* y, void* stream);

/* ---------------------------------------------------------------------------
 * Sensitivity (hyper.ai summary, Method, Eq. 14: s = tr(H_G) tr(H_X) computed
 * after BiIP).  out3 (device, 3 doubles) = { tr(HX), tr(HG), tr(HX) * tr(HG) },
 * diagonals summed in fp64.  HX is n x n, HG is m x m (fp32 device).
 * ------------------------------------------------------------------------- */
kronq_status kronq_sensitivity(const float* HX, int64_t n, int64_t ldhx, const float* HG,
                               int64_t m, int64_t ldhg, double* out3, void* stream);

/* ---------------------------------------------------------------------------
 * Bit allocation (hyper.ai summary, Method: higher bit-widths for larger
 * s; GitHub README, --inter_layer_mp: upgrade the most sensitive sublayers by
 * +1 bit).  Host only, pure, deterministic.  Every sublayer starts at bmin;
 * sublayers are visited by descending score (ties: lower index first) and each
 * is raised one bit at a time while it is below bmax and
 * sum(bits * n_params) stays <= budget_bits.  scores (L doubles), n_params
 * (L int64 > 0) and bits_out (L int32) are host arrays.
 * KRONQ_EINVAL if L < 1, bmin < 1, bmax < bmin, a score is NaN or
 * budget_bits < bmin * sum(n_params).
 * ------------------------------------------------------------------------- */
kronq_status kronq_allocate_bits(int32_t L, const double* scores, const int64_t* n_params,
                                 int32_t bmin, int32_t bmax, int64_t budget_bits,
                                 int32_t* bits_out);

/* ---------------------------------------------------------------------------
 * Allocation variants (hyper.ai summary, Method: a sublayer's expected loss is
 * proportional to eps^2 tr(H) with tr(H) = tr(H_X) tr(H_G), so higher
 * bit-widths go to larger scores; GitHub README, --inter_layer_mp N: upgrade
 * the top-N sensitive sublayer types by +1 bit).  Host only, pure,
 * deterministic; arguments and errors as kronq_allocate_bits.
 *
 * kronq_allocate_bits_passwise: every sublayer starts at bmin; whole passes
 *   over the sublayers in descending score order (ties: lower index) give each
 *   +1 bit while it is below bmax and sum(bits * n_params) stays <= budget_bits,
 *   until a pass changes nothing.
 * kronq_allocate_bits_marginal: with eps(b) ~ 2^-b (a uniform grid's step
 *   halves with each bit), one more bit lowers sublayer i's loss in proportion
 *   to s_i 4^-b_i at a cost of n_params[i] bits.  Repeatedly apply, among the
 *   upgrades that fit, the one with the largest ldexp(s_i, -2 b_i) / n_params[i]
 *   (ties: lower index), until none fits.
 * ------------------------------------------------------------------------- */
kronq_status kronq_allocate_bits_passwise(int32_t L, const double* scores,
                                          const int64_t* n_params, int32_t bmin, int32_t bmax,
                                          int64_t budget_bits, int32_t* bits_out);
kronq_status kronq_allocate_bits_marginal(int32_t L, const double* scores,
                                          const int64_t* n_params, int32_t bmin, int32_t bmax,
                                          int64_t budget_bits, int32_t* bits_out);

/* Type-level allocation (GitHub README, --inter_layer_mp N).  Sublayer i has
 * type type_of[i] in [0, n_types) (e.g. q, k, v, o, gate, up, down across all
 * layers); a type's score is the sum of its sublayers' scores (added in
 * ascending sublayer order).  The n_upgrade types with the largest sums (ties:
 * lower type id) get base_bits + 1, the others base_bits; bits_out[i] is
 * sublayer i's width.  KRONQ_EINVAL for L < 1, n_types < 1, a type outside
 * [0, n_types), base_bits outside 1..63, n_upgrade outside [0, n_types] or a
 * NaN score.  Host arrays. */
kronq_status kronq_allocate_types(int32_t L, const double* scores, const int32_t* type_of,
                                  int32_t n_types, int32_t base_bits, int32_t n_upgrade,
                                  int32_t* bits_out);

#ifdef __cplusplus
}
#endif

#endif /* KRONQ_H */
