// Weight diagnostics of incoherence processing (Pith review, Figure 2: CV_in
// and CV_out, the coefficients of variation of the column norms and of the
// row norms of W; incoherence on the input side alone leaves the row norms,
// and so CV_out, in place, while BiIP lowers both).
//
//   cv_partial  one workgroup per tile of 64 rows x 1024 columns, walked as
//               four groups of 16 rows: a thread holds a float4 of each of the
//               16 rows of a group (16 loads in flight, the next group's loads
//               issued before this group's sums), squares and sums them down
//               its columns and, through DPP and LDS, along each row.  Partial
//               column sums per row block and partial row sums per column
//               block go to the workspace.  This pass reads W once and carries
//               all of its bytes (HBM-bound).
//   cv_norms    sums the partials in fp64 and takes square roots: the n column
//               norms and the m row norms; each workgroup also writes the fp64
//               sums of its norms and of their squares, per set.
//   cv_final    adds those sums: mean and population variance of each set of
//               norms as E[x] and E[x^2] - E[x]^2 in fp64 (the cancellation
//               costs 2^-52 / CV^2 relative, below 1e-8 for CV >= 1e-4),
//               CV = std / mean.
#include <algorithm>
#include <cmath>

#include "kronq_internal.h"

namespace kronq {
namespace {

constexpr int NT = 256;
constexpr int RG = 16;     // rows of a group (loads in flight per thread)
constexpr int RB = 64;     // rows of a tile
constexpr int CB = 1024;   // columns of a tile (a float4 per thread)

template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                   CTRL, ROWS, 0xF, false));
}

// wave sum in lane 63 (quad and row butterflies, then the row broadcasts)
__device__ __forceinline__ float wave_total(float v) {
  v = dpp_add<0xB1>(v);
  v = dpp_add<0x4E>(v);
  v = dpp_add<0x141>(v);
  v = dpp_add<0x140>(v);
  v = dpp_add<0x142, 0xA>(v);
  v = dpp_add<0x143, 0xC>(v);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Loads read clamped, always valid addresses and discard what lies outside the
// matrix with a select (VEC: n and ldw multiples of 4, W 16-byte aligned).
template <bool VEC>
__device__ __forceinline__ void load_group(const float* __restrict__ W, int64_t m, int64_t n,
                                           int64_t ldw, int64_t r0, int64_t c0, float4 (&x)[RG]) {
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    const int64_t row = r0 + r;
    const int64_t rr = row < m ? row : 0;
    if (VEC) {
      const int64_t cc = c0 < n ? c0 : 0;
      const float4 v = *reinterpret_cast<const float4*>(W + rr * ldw + cc);
      const bool in = row < m && c0 < n;
      x[r] = in ? v : make_float4(0.f, 0.f, 0.f, 0.f);
    } else {
      float e[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t c = c0 + j;
        const float v = W[rr * ldw + (c < n ? c : 0)];
        e[j] = (row < m && c < n) ? v : 0.f;
      }
      x[r] = make_float4(e[0], e[1], e[2], e[3]);
    }
  }
}

template <bool VEC>
__global__ void __launch_bounds__(NT) cv_partial(const float* __restrict__ W, int64_t m, int64_t n,
                                                 int64_t ldw, int64_t nrb, float* __restrict__ colpart,
                                                 float* __restrict__ rowpart) {
  __shared__ float red[2][NT / 64][RG];
  const int64_t rb = blockIdx.x % nrb, cb = blockIdx.x / nrb;
  const int64_t r0 = rb * RB;
  const int64_t c0 = cb * CB + 4 * threadIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float4 col = make_float4(0.f, 0.f, 0.f, 0.f);
  float4 a[RG], b[RG];
  load_group<VEC>(W, m, n, ldw, r0, c0, a);
#pragma unroll
  for (int grp = 0; grp < RB / RG; ++grp) {
    float4 (&x)[RG] = (grp & 1) ? b : a;
    if (grp + 1 < RB / RG) load_group<VEC>(W, m, n, ldw, r0 + (grp + 1) * RG, c0, (grp & 1) ? a : b);
    float rowsq[RG];
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      const float4 v = x[r];
      col.x = fmaf(v.x, v.x, col.x);
      col.y = fmaf(v.y, v.y, col.y);
      col.z = fmaf(v.z, v.z, col.z);
      col.w = fmaf(v.w, v.w, col.w);
      rowsq[r] = fmaf(v.x, v.x, fmaf(v.y, v.y, fmaf(v.z, v.z, v.w * v.w)));
    }
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      const float t = wave_total(rowsq[r]);
      if (lane == 0) red[grp & 1][wave][r] = t;
    }
    __syncthreads();   // the other buffer's readers finished one group ago
    const int64_t row = r0 + grp * RG + threadIdx.x;
    if (threadIdx.x < RG && row < m) {
      float t = 0.f;
#pragma unroll
      for (int w = 0; w < NT / 64; ++w) t += red[grp & 1][w][threadIdx.x];
      rowpart[cb * m + row] = t;
    }
  }
  const float cv[4] = {col.x, col.y, col.z, col.w};
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (c0 + j < n) colpart[rb * n + c0 + j] = cv[j];
}

// norms[j] = sqrt(sum_b part[b * len + j]) for j < len, summed in fp64; the
// workgroup's sums of norms and squared norms (columns, rows) go to sums[4 * wg]
__global__ void __launch_bounds__(NT) cv_norms(const float* __restrict__ colpart, int64_t nrb,
                                               int64_t n, const float* __restrict__ rowpart,
                                               int64_t ncb, int64_t m, float* __restrict__ coln,
                                               float* __restrict__ rown, double* __restrict__ sums) {
  __shared__ double red[NT / 64][4];
  const int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x;
  double v[4] = {0.0, 0.0, 0.0, 0.0};   // column sum, column squares, row sum, row squares
  if (i < n) {
    double s = 0.0;
#pragma unroll 8
    for (int64_t b = 0; b < nrb; ++b) s += colpart[b * n + i];
    const float c = (float)std::sqrt(s);
    coln[i] = c;
    v[0] = c;
    v[1] = (double)c * c;
  } else if (i < n + m) {
    const int64_t r = i - n;
    double s = 0.0;
#pragma unroll 8
    for (int64_t b = 0; b < ncb; ++b) s += rowpart[b * m + r];
    const float c = (float)std::sqrt(s);
    rown[r] = c;
    v[2] = c;
    v[3] = (double)c * c;
  }
#pragma unroll
  for (int k = 0; k < 4; ++k)
    for (int off = 32; off > 0; off >>= 1) v[k] += __shfl_xor(v[k], off);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0)
#pragma unroll
    for (int k = 0; k < 4; ++k) red[wave][k] = v[k];
  __syncthreads();
  if (threadIdx.x < 4) {
    double t = 0.0;
    for (int w = 0; w < NT / 64; ++w) t += red[w][threadIdx.x];
    sums[4 * blockIdx.x + threadIdx.x] = t;
  }
}

// out[0] = CV of the column norms (n), out[1] = CV of the row norms (m)
__global__ void __launch_bounds__(64) cv_final(const double* __restrict__ sums, int64_t nwg,
                                               int64_t n, int64_t m, double* __restrict__ out) {
  double v[4] = {0.0, 0.0, 0.0, 0.0};
  for (int64_t w = threadIdx.x; w < nwg; w += 64)
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] += sums[4 * w + k];
#pragma unroll
  for (int k = 0; k < 4; ++k)
    for (int off = 32; off > 0; off >>= 1) v[k] += __shfl_xor(v[k], off);
  if (threadIdx.x == 0) {
    for (int set = 0; set < 2; ++set) {
      const double len = (double)(set ? m : n);
      const double mean = v[2 * set] / len;
      const double var = v[2 * set + 1] / len - mean * mean;
      out[set] = std::sqrt(var > 0.0 ? var : 0.0) / mean;
    }
  }
}

struct CvLayout {
  int64_t nrb, ncb;
  size_t colpart, rowpart, coln, rown, sums, total;   // byte offsets and size
};

CvLayout cv_layout(int64_t m, int64_t n) {
  CvLayout L{};
  L.nrb = (m + RB - 1) / RB;
  L.ncb = (n + CB - 1) / CB;
  L.colpart = 0;
  L.rowpart = align_up((size_t)L.nrb * (size_t)n * sizeof(float), 256);
  L.coln = L.rowpart + align_up((size_t)L.ncb * (size_t)m * sizeof(float), 256);
  L.rown = L.coln + align_up((size_t)n * sizeof(float), 256);
  L.sums = L.rown + align_up((size_t)m * sizeof(float), 256);
  L.total = L.sums + align_up((size_t)((n + m + NT - 1) / NT) * 4 * sizeof(double), 256);
  return L;
}

// ---------------------------------------------------------------- finiteness

// an fp32 value is NaN or infinite exactly when its exponent field is all ones
__device__ __forceinline__ bool nonfinite_bits(float v) {
  return (__float_as_uint(v) & 0x7f800000u) == 0x7f800000u;
}

__global__ void finite_clear(int32_t* flag) { *flag = 0; }

// grid-stride scan; any thread that meets a non-finite value stores 1 (all
// such stores write the same value, so their order does not matter)
__global__ void __launch_bounds__(256) finite_scan(const float* __restrict__ A, int64_t rows,
                                                   int64_t cols, int64_t ld, int32_t* flag) {
  bool bad = false;
  const int64_t total = rows * cols;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / cols, c = i - r * cols;
    bad |= nonfinite_bits(A[r * ld + c]);
  }
  if (bad) *flag = 1;
}

}  // namespace

kronq_status finite_launch(const float* A, int64_t rows, int64_t cols, int64_t ld, int32_t* flag,
                           hipStream_t s) {
  hipLaunchKernelGGL(finite_clear, dim3(1), dim3(1), 0, s, flag);
  KQ_LAUNCHED("finite_clear");
  if (rows == 0 || cols == 0) return KRONQ_OK;
  const int64_t total = rows * cols;
  const unsigned grid = (unsigned)std::min<int64_t>((total + 255) / 256, 8192);
  hipLaunchKernelGGL(finite_scan, dim3(grid), dim3(256), 0, s, A, rows, cols, ld, flag);
  KQ_LAUNCHED("finite_scan");
  return KRONQ_OK;
}

size_t cv_ws_bytes(int64_t m, int64_t n) { return cv_layout(m, n).total; }

kronq_status cv_launch(const float* W, int64_t m, int64_t n, int64_t ldw, double* out2,
                       float* col_norms, float* row_norms, void* ws, hipStream_t s) {
  const CvLayout L = cv_layout(m, n);
  char* base = static_cast<char*>(ws);
  float* colpart = reinterpret_cast<float*>(base + L.colpart);
  float* rowpart = reinterpret_cast<float*>(base + L.rowpart);
  float* coln = col_norms ? col_norms : reinterpret_cast<float*>(base + L.coln);
  float* rown = row_norms ? row_norms : reinterpret_cast<float*>(base + L.rown);
  const int64_t tiles = L.nrb * L.ncb;
  if (tiles > 0x7fffffff) return fail(KRONQ_EINVAL, "kronq_weight_cv: matrix too large");
  const bool vec = n % 4 == 0 && ldw % 4 == 0 && reinterpret_cast<uintptr_t>(W) % 16 == 0;
  if (vec)
    hipLaunchKernelGGL(cv_partial<true>, dim3((unsigned)tiles), dim3(NT), 0, s, W, m, n, ldw, L.nrb,
                       colpart, rowpart);
  else
    hipLaunchKernelGGL(cv_partial<false>, dim3((unsigned)tiles), dim3(NT), 0, s, W, m, n, ldw,
                       L.nrb, colpart, rowpart);
  KQ_LAUNCHED("cv_partial");
  double* sums = reinterpret_cast<double*>(base + L.sums);
  const int64_t nwg = (n + m + NT - 1) / NT;
  hipLaunchKernelGGL(cv_norms, dim3((unsigned)nwg), dim3(NT), 0, s, colpart, L.nrb, n, rowpart,
                     L.ncb, m, coln, rown, sums);
  KQ_LAUNCHED("cv_norms");
  hipLaunchKernelGGL(cv_final, dim3(1), dim3(64), 0, s, sums, nwg, n, m, out2);
  KQ_LAUNCHED("cv_final");
  return KRONQ_OK;
}

}  // namespace kronq
