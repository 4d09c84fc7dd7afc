// GPTAQ asymmetric correction of the column loop (Pith review of the KronQ
// paper, Algorithm 2: P = alpha (dXX^T L) (.) M_U L^T after the inverse
// Cholesky step, used by the column loop; hyper.ai summary, Method: the
// objective corrects for input drift by asymmetric calibration, and the
// column update after quantizing column p carries the scaled quantization
// error and P).
//
// With R the upper factor (R^T R = Hd^-1, processing order) the pages' lower
// factor is L = R^T, so
//   K = C_p R^T            C_p = C[perm][:, perm], C = (X_fp - X)^T X / N
//                          (the drift term, rotated by the input side of BiIP)
//   P = alpha triu1(K) R   triu1: the strictly upper part
// and in the column loop every later column k moves by + w_j P[j][k] once
// column j is quantized, w_j the full-precision weight of column j.  That
// drift shift depends on W and P alone, so it is formed up front as two
// products:
//   X1[r][k] = sum over j in units before k's unit of Wp[r][j] P[j][k]
//   X2[r][k] = sum over j < k in k's unit of Wp[r][j] P[j][k]
// (a unit is a quantization group, or a 128-column block of the loop for one
// grid per row; Wp = W in processing order).  X1 enters the loop's start
// values (W + X1 is what the product waves read), so the grid of a group sees
// the drift of every earlier unit; X2 is added to a unit's values right after
// its grid is taken.
//
// All three products run on one tiled kernel: fp32 in and out on
// v_mfma_f32_32x32x2f32, a 128 x 128 output tile per workgroup (four waves as
// 2 x 2, each 64 x 64 as 2 x 2 accumulators of 32 x 32), K staged 16 at a time
// through LDS with the next stage's global loads in registers while the
// current stage is multiplied.  The triangular structure sets each tile's K
// range (and skips tiles that are known to be zero).
#include <algorithm>

#include "kronq_internal.h"

namespace kronq {
namespace {

typedef float f32x16_t __attribute__((__vector_size__(16 * sizeof(float))));

constexpr int GT = 128;      // output tile edge
constexpr int GK = 16;       // K per stage
constexpr int GLD = GT + 4;  // padded LDS row (floats)

enum KRange { K_FROM_COL, K_ROW_TO_COL, K_ZERO_TO_COL, K_COL_TO_COL };
enum BMask { B_ALL, B_UNIT_BEFORE, B_UNIT_SAME_BELOW };

struct GemmArgs {
  const float* A;        // rows x K, row-major (row and column gathers optional)
  int64_t lda;
  const int32_t* arow;   // A row r = A[arow[r]] (NULL: r)
  const int32_t* acol;   // A column k = A[.][acol[k]] (NULL: k)
  const float* B;        // NN: K x cols, NT: cols x K (row-major)
  int64_t ldb;
  float* C;              // rows x cols output
  int64_t ldc;
  const int32_t* ccol;   // output column c goes to C[.][ccol[c]] (NULL: c)
  const float* base;     // C = base + alpha acc (same column map; NULL: no base)
  int64_t ldbase;
  int64_t rows, cols, K;
  float alpha;
  int unit;              // B masks: the unit length
  int tiles_c;           // tile columns
};

__device__ __forceinline__ int64_t gather(const int32_t* map, int64_t i) { return map ? (int64_t)map[i] : i; }

template <bool NT, int KR, int BM, bool SKIP_LOWER, bool ZERO_LOWER, bool STRICT_UPPER_OUT>
__global__ void __launch_bounds__(256) gemm_tile(GemmArgs g) {
  __shared__ float As[GK][GLD];
  __shared__ float Bs[GK][GLD];
  const int tr = blockIdx.x / g.tiles_c, tc = blockIdx.x % g.tiles_c;
  const int64_t r0 = (int64_t)tr * GT, c0 = (int64_t)tc * GT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lk = lane >> 5;
  const bool lower = tc < tr;
  if (SKIP_LOWER && lower) return;
  int64_t klo = 0, khi = g.K;
  if (KR == K_FROM_COL) klo = c0;
  if (KR == K_ROW_TO_COL) { klo = r0; khi = std::min<int64_t>(g.K, c0 + GT); }
  if (KR == K_ZERO_TO_COL) khi = std::min<int64_t>(g.K, c0 + GT);
  if (KR == K_COL_TO_COL) { klo = c0; khi = std::min<int64_t>(g.K, c0 + GT); }
  f32x16_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

  const bool compute = !(ZERO_LOWER && lower) && klo < khi;
  if (compute) {
    float ra[8], rb[8];
    // stage loads: A tile 128 x 16 (element e: row e / 16, k e % 16), B tile
    // 16 x 128 (NN: k e / 128, column e % 128; NT: column e / 16, k e % 16)
    auto load = [&](int64_t k0) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int e = tid + 256 * q;
        {
          const int i = e >> 4, k = e & 15;
          const int64_t rr = r0 + i, kk = k0 + k;
          ra[q] = (rr < g.rows && kk < khi) ? g.A[gather(g.arow, rr) * g.lda + gather(g.acol, kk)] : 0.f;
        }
        int j, k;
        if (NT) { j = e >> 4; k = e & 15; } else { k = e >> 7; j = e & 127; }
        const int64_t cc = c0 + j, kk = k0 + k;
        float v = 0.f;
        if (cc < g.cols && kk < khi) {
          bool keep = true;
          if (BM == B_UNIT_BEFORE) keep = kk / g.unit < cc / g.unit;
          if (BM == B_UNIT_SAME_BELOW) keep = kk / g.unit == cc / g.unit && kk < cc;
          if (keep) v = NT ? g.B[cc * g.ldb + kk] : g.B[kk * g.ldb + cc];
        }
        rb[q] = v;
      }
    };
    auto store = [&]() {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int e = tid + 256 * q;
        As[e & 15][e >> 4] = ra[q];
        if (NT) Bs[e & 15][e >> 4] = rb[q];
        else Bs[e >> 7][e & 127] = rb[q];
      }
    };
    load(klo);
    store();
    __syncthreads();
    for (int64_t k0 = klo; k0 < khi; k0 += GK) {
      const bool more = k0 + GK < khi;
      if (more) load(k0 + GK);
#pragma unroll
      for (int kk = 0; kk < GK; kk += 2) {
        float af[2], bf[2];
#pragma unroll
        for (int a = 0; a < 2; ++a) af[a] = As[kk + lk][wm * 64 + 32 * a + lr];
#pragma unroll
        for (int b = 0; b < 2; ++b) bf[b] = Bs[kk + lk][wn * 64 + 32 * b + lr];
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 2; ++b)
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[a], bf[b], acc[a][b], 0, 0, 0);
      }
      __syncthreads();
      if (more) {
        store();
        __syncthreads();
      }
    }
  }
  // 32 x 32 accumulator: lane holds column lr; register v holds row
  // 8 (v / 4) + 4 lk + v % 4
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t r = r0 + wm * 64 + 32 * a + 8 * (v >> 2) + 4 * lk + (v & 3);
        const int64_t c = c0 + wn * 64 + 32 * b + lr;
        if (r >= g.rows || c >= g.cols) continue;
        float x = g.alpha * acc[a][b][v];
        if (STRICT_UPPER_OUT && c <= r) x = 0.f;
        const int64_t oc = gather(g.ccol, c);
        if (g.base) x += g.base[r * g.ldbase + oc];
        g.C[r * g.ldc + oc] = x;
      }
}

template <bool NT, int KR, int BM, bool SKIP_LOWER, bool ZERO_LOWER, bool SU>
kronq_status run_gemm(GemmArgs g, hipStream_t s, const char* name) {
  g.tiles_c = (int)((g.cols + GT - 1) / GT);
  const int64_t tiles = ((g.rows + GT - 1) / GT) * (int64_t)g.tiles_c;
  if (tiles > 0x7fffffff) return fail(KRONQ_EINVAL, "%s: matrix too large", name);
  if (tiles == 0) return KRONQ_OK;
  hipLaunchKernelGGL((gemm_tile<NT, KR, BM, SKIP_LOWER, ZERO_LOWER, SU>), dim3((unsigned)tiles), dim3(256), 0,
                     s, g);
  KQ_LAUNCHED(name);
  return KRONQ_OK;
}

// dX = X_fp - X (exact in fp32: both are bf16) as hi + lo, each bf16: hi =
// bf16(dX), lo = bf16(dX - hi); the pair carries 16 significant bits, which is
// dX exactly unless X_fp and X differ by more than a factor 2^8.
__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

__global__ void __launch_bounds__(256) drift_split(const uint16_t* __restrict__ Xfp,
                                                   const uint16_t* __restrict__ X, int64_t rows, int64_t n,
                                                   int64_t ld, uint16_t* __restrict__ hi,
                                                   uint16_t* __restrict__ lo) {
  const int64_t total = rows * n;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / n, c = i - r * n;
    const float a = __uint_as_float((uint32_t)Xfp[r * ld + c] << 16);
    const float b = __uint_as_float((uint32_t)X[r * ld + c] << 16);
    const float d = a - b;
    const uint16_t h = bf16_rne(d);
    const float hf = __uint_as_float((uint32_t)h << 16);
    hi[i] = h;
    lo[i] = bf16_rne(d - hf);
  }
}

constexpr int64_t kDriftChunk = 32768;   // tokens per chunk of the drift term

}  // namespace

// C = (X_fp - X)^T X / N in token chunks: each chunk's dX is split into two
// bf16 matrices, and C accumulates hi^T X + lo^T X on the bf16 matrix cores
// (the cross-product tiles with beta = 1 after the first call).  Forming dX
// first keeps the fp32 accumulation on the drift's own scale; X_fp^T X - H_X
// would cancel most of the fp32 sums.
size_t drift_cross_ws_bytes(int64_t N, int64_t n) {
  const int64_t ch = std::min<int64_t>(N, kDriftChunk);
  return 2 * align_up((size_t)ch * (size_t)n * sizeof(uint16_t), 256) + gram_cross_ws_bytes(ch, n);
}

kronq_status drift_cross_launch(const void* Xfp, const void* X, int64_t N, int64_t n, int64_t ld, float* C,
                                int64_t ldc, void* ws, hipStream_t s) {
  const int64_t ch = std::min<int64_t>(N, kDriftChunk);
  const size_t half = align_up((size_t)ch * (size_t)n * sizeof(uint16_t), 256);
  uint16_t* hi = static_cast<uint16_t*>(ws);
  uint16_t* lo = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + half);
  void* cws = static_cast<char*>(ws) + 2 * half;
  const float scale = (float)(1.0 / (double)N);
  for (int64_t t0 = 0; t0 < N; t0 += ch) {
    const int64_t rows = std::min<int64_t>(ch, N - t0);
    const uint16_t* a = static_cast<const uint16_t*>(Xfp) + t0 * ld;
    const uint16_t* b = static_cast<const uint16_t*>(X) + t0 * ld;
    const unsigned grid = (unsigned)std::min<int64_t>((rows * n + 255) / 256, 16384);
    hipLaunchKernelGGL(drift_split, dim3(grid), dim3(256), 0, s, a, b, rows, n, ld, hi, lo);
    KQ_LAUNCHED("drift_split");
    kronq_status st = gram_cross_launch(hi, b, rows, n, n, C, ldc, scale, t0 == 0 ? 0.0f : 1.0f, nullptr, 0,
                                        cws, s);
    if (st) return st;
    st = gram_cross_launch(lo, b, rows, n, n, C, ldc, scale, 1.0f, nullptr, 0, cws, s);
    if (st) return st;
  }
  return KRONQ_OK;
}

size_t gptaq_correction_ws_bytes(int64_t n) { return align_up((size_t)n * (size_t)n * sizeof(float), 256); }

kronq_status gptaq_correction_launch(const float* C, int64_t n, int64_t ldc, const float* R, int64_t ldr,
                                     const int32_t* perm, float alpha, float* P, int64_t ldp, void* ws,
                                     hipStream_t s) {
  float* K = static_cast<float*>(ws);   // n x n: triu1(C_p R^T), tiles on and above the diagonal
  GemmArgs g{};
  g.A = C;
  g.lda = ldc;
  g.arow = perm;
  g.acol = perm;
  g.B = R;
  g.ldb = ldr;
  g.C = K;
  g.ldc = n;
  g.rows = n;
  g.cols = n;
  g.K = n;
  g.alpha = 1.0f;
  g.unit = 1;
  // K[j][i] = sum_{l >= i} C_p[j][l] R[i][l]  (R[i][l] = 0 for l < i)
  kronq_status st = run_gemm<true, K_FROM_COL, B_ALL, true, false, true>(g, s, "gptaq_k");
  if (st) return st;
  GemmArgs h{};
  h.A = K;
  h.lda = n;
  h.B = R;
  h.ldb = ldr;
  h.C = P;
  h.ldc = ldp;
  h.rows = n;
  h.cols = n;
  h.K = n;
  h.alpha = alpha;
  h.unit = 1;
  // P[j][k] = alpha sum_{j < i <= k} K[j][i] R[i][k]; tiles below the diagonal are zero
  return run_gemm<false, K_ROW_TO_COL, B_ALL, false, true, false>(h, s, "gptaq_p");
}

size_t gptaq_shift_ws_bytes(int64_t m, int64_t n) {
  return 2 * align_up((size_t)m * (size_t)n * sizeof(float), 256);
}

kronq_status gptaq_shift_launch(const float* W, int64_t m, int64_t n, int64_t ldw, const int32_t* perm,
                                const float* P, int64_t ldp, int unit, float* W1, float* X2,
                                hipStream_t s) {
  GemmArgs g{};
  g.A = W;
  g.lda = ldw;
  g.acol = perm;
  g.B = P;
  g.ldb = ldp;
  g.C = W1;
  g.ldc = n;
  g.ccol = perm;
  g.base = W;
  g.ldbase = ldw;
  g.rows = m;
  g.cols = n;
  g.K = n;
  g.alpha = 1.0f;
  g.unit = unit;
  // W1[r][perm[k]] = W[r][perm[k]] + sum over earlier units' j of Wp[r][j] P[j][k]
  kronq_status st = run_gemm<false, K_ZERO_TO_COL, B_UNIT_BEFORE, false, false, false>(g, s, "gptaq_x1");
  if (st) return st;
  GemmArgs h = g;
  h.C = X2;
  h.ldc = n;
  h.ccol = nullptr;
  h.base = nullptr;
  // X2[r][k] = sum over j < k in k's unit of Wp[r][j] P[j][k] (processing order)
  return run_gemm<false, K_COL_TO_COL, B_UNIT_SAME_BELOW, false, false, false>(h, s, "gptaq_x2");
}

}  // namespace kronq
