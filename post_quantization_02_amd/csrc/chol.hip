// Act-order, damping and the inverse Cholesky factor of H_X (Pith review of
// the KronQ paper, Algorithm 2: the damped H_X is H_X + lambda mean(diag) I
// and the column loop uses its inverse Cholesky factor; GitHub README,
// --act_order).
//
// R is the upper triangular factor with positive diagonal and R^T R = Hd^-1,
// Hd = P (H + damp I) P^T.  With J the exchange matrix, factor the reversed
// matrix A = J Hd J = L L^T (L lower); then Hd = (J L J)(J L J)^T with J L J
// upper, so Hd^-1 = (J L^-1 J)^T (J L^-1 J) and R = J L^-1 J.  This needs one
// factorization and one triangular inverse (2 n^3 / 3 flops).
//
// Blocked right-looking sweep over panels of NB = 128 columns of A (padded
// with an identity block to a multiple of NB; the padding is block diagonal
// with A so it changes nothing), solving L Y = I alongside (B starts as I):
//   diag kernel   (1 workgroup, 512 threads): Cholesky of A_pp and, in the
//                 same elimination sweep, Linv_pp (augmented [A_pp | I]); fp64
//                 in registers, 8 x 8 elements per thread, 2 barriers per
//                 column; pivots <= 0 are reported
//   panel kernel  : Lp_i = A_ip Linv_pp^T (i > p) and Yp_c = Linv_pp B_pc
//                   (c <= p), each as four 128 x 32 quarter tiles
//   update kernel : A_ij -= Lp_i Lp_j^T (i >= j > p; Cholesky SYRK),
//                   B_ic -= Lp_i Yp_c   (i > p, c <= p; forward substitution),
//                   B_pc  = Yp_c        (row block p of Y = L^-1 is final)
// and finally R = J Y J.  Tile products run on the fp32 matrix cores
// (v_mfma_f32_32x32x2f32).  A device flag set by a failed pivot makes every
// later kernel return at once; the host reads the flag after the last launch.
#include "kronq_internal.h"

namespace kronq {
namespace {

typedef float f32x16_t __attribute__((__vector_size__(16 * sizeof(float))));

constexpr int NB = 128;
constexpr int KS = 32;        // K rows per LDS stage
constexpr int LDT = NB + 1;   // odd LDS stride: conflict-free transposed stores

struct CholWs {
  float* A;       // npad x npad (reversed, permuted, damped)
  float* B;       // npad x npad (forward substitution; ends as Y = L^-1)
  float* Lp;      // npad x NB   (panel L_ip of the current step)
  float* Yp;      // NB x npad   (row block Y_p of the current step)
  float* Linv;    // NB x NB     (inverse of the current diagonal block)
  double* damp;   // lambda * mean(diag H)
  int* flag;      // nonzero after a failed pivot
  long long* info;
};

size_t ws_layout(int64_t n, CholWs* w, void* base) {
  const int64_t npad = (n + NB - 1) / NB * NB;
  const size_t sA = align_up((size_t)npad * npad * sizeof(float), 256);
  const size_t sP = align_up((size_t)npad * NB * sizeof(float), 256);
  size_t off = 0;
  char* b = static_cast<char*>(base);
  if (w) w->A = reinterpret_cast<float*>(b + off);
  off += sA;
  if (w) w->B = reinterpret_cast<float*>(b + off);
  off += sA;
  if (w) w->Lp = reinterpret_cast<float*>(b + off);
  off += sP;
  if (w) w->Yp = reinterpret_cast<float*>(b + off);
  off += sP;
  if (w) w->Linv = reinterpret_cast<float*>(b + off);
  off += align_up((size_t)NB * NB * sizeof(float), 256);
  if (w) w->damp = reinterpret_cast<double*>(b + off);
  off += 256;
  if (w) w->flag = reinterpret_cast<int*>(b + off);
  off += 256;
  if (w) w->info = reinterpret_cast<long long*>(b + off);
  off += 256;
  return off;
}

// ------------------------------------------------------------------ prep

__global__ void __launch_bounds__(256) chol_prep(const float* H, int64_t n, int64_t ldh, float lambda,
                                                 CholWs w) {
  __shared__ double red[4];
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += 256) acc += (double)H[i * ldh + i];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    const double tr = red[0] + red[1] + red[2] + red[3];
    *w.damp = (double)lambda * (tr / (double)n);
    *w.flag = 0;
    *w.info = -1;
  }
}

// perm = stable descending order of diag(H): rank(i) = #{j : d_j > d_i} +
// #{j < i : d_j == d_i}; perm[rank(i)] = i.
__global__ void __launch_bounds__(256) chol_act_order(const float* H, int64_t n, int64_t ldh,
                                                      int32_t* perm) {
  __shared__ float chunk[1024];
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const float di = (i < n) ? H[i * ldh + i] : 0.f;
  const bool ni = isnan(di);
  int64_t rank = 0;
  for (int64_t j0 = 0; j0 < n; j0 += 1024) {
    __syncthreads();
    for (int q = threadIdx.x; q < 1024; q += 256)
      chunk[q] = (j0 + q < n) ? H[(j0 + q) * ldh + (j0 + q)] : 0.f;
    __syncthreads();
    const int cnt = (int)min<int64_t>(1024, n - j0);
    for (int q = 0; q < cnt; ++q) {
      // strict total order: larger first, NaN last, ties by index
      const float dj = chunk[q];
      const bool nj = isnan(dj);
      const bool before = (nj || ni) ? (nj && ni ? (j0 + q < i) : ni) : (dj > di || (dj == di && j0 + q < i));
      rank += before;
    }
  }
  if (i < n) perm[rank] = (int32_t)i;
}

__global__ void chol_identity_perm(int64_t n, int32_t* perm) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) perm[i] = (int32_t)i;
}

// A[a][b] = H[perm[n-1-a]][perm[n-1-b]] + damp [a == b]  (identity padding);
// B = I.
__global__ void __launch_bounds__(256) chol_gather(const float* H, int64_t n, int64_t ldh,
                                                   const int32_t* perm, int64_t npad, CholWs w) {
  const int64_t a = blockIdx.y;
  const float damp = (float)*w.damp;
  for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < npad; b += (int64_t)gridDim.x * 256) {
    float v;
    if (a < n && b < n) {
      const int64_t r = min<int64_t>(max<int32_t>(perm[n - 1 - a], 0), n - 1);
      const int64_t c = min<int64_t>(max<int32_t>(perm[n - 1 - b], 0), n - 1);
      v = H[r * ldh + c];
      if (a == b) v += damp;
    } else {
      v = (a == b) ? 1.f : 0.f;
    }
    w.A[a * npad + b] = v;
    w.B[a * npad + b] = (a == b) ? 1.f : 0.f;
  }
}

// ------------------------------------------------------- diagonal block

// Row-block of the 8 x 8 element block held by a thread: the four waves of a
// role take row blocks {w, 7-w, 8+w, 15-w} so that the lower-triangle work is
// even across waves.
__device__ __forceinline__ int diag_rowblock(int w, int r) {
  return r == 0 ? w : r == 1 ? 7 - w : r == 2 ? 8 + w : 15 - w;
}

// Factor A_pp = L L^T and invert L in one elimination sweep over [A_pp | I]:
// for each column j, l_jj = sqrt(a_jj), l_ij = a_ij / l_jj (i > j), row j of
// the right-hand side becomes x_j = b_j / l_jj, then a_ik -= l_ij l_kj and
// b_ic -= l_ij x_jc for i > j.  Threads 0..255 hold 8 x 8 blocks of A, threads
// 256..511 the blocks of B (= L^-1 at the end), fp64 in registers.
__global__ void __launch_bounds__(512) chol_diag(int64_t npad, int64_t n, int p, CholWs w) {
  if (*w.flag) return;
  __shared__ double col[NB];
  __shared__ double xrow[NB];
  __shared__ double piv;
  __shared__ int bad;
  const int tid = threadIdx.x;
  const bool isA = tid < 256;
  const int t = tid & 255;
  const int wv = t >> 6, ln = t & 63;
  const int bi = diag_rowblock(wv, ln >> 4);  // row block
  const int bk = ln & 15;                     // column block
  const bool act = bk <= bi;                  // lower-triangle block
  double r[8][8];
  const float* Ap = w.A + (int64_t)p * NB * npad + (int64_t)p * NB;
  if (isA) {
#pragma unroll
    for (int ii = 0; ii < 8; ++ii)
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        r[ii][kk] = act ? (double)Ap[(int64_t)(8 * bi + ii) * npad + 8 * bk + kk] : 0.0;
  } else {
#pragma unroll
    for (int ii = 0; ii < 8; ++ii)
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) r[ii][kk] = (bi == bk && ii == kk) ? 1.0 : 0.0;
  }
  if (tid == 0) {
    piv = r[0][0];
    bad = -1;
  }
  __syncthreads();
  // The broadcast column (l_ij, zero for i <= j) and row (x_jc, zero for
  // c > j) make every update below uniform: each thread updates its whole
  // 8 x 8 block; entries outside the trailing region receive zero, and the
  // upper blocks that take part are never read.
  for (int jb = 0; jb < NB / 8; ++jb) {
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int j = 8 * jb + jj;
      // ---- column j of L and row j of L^-1
      const double d = piv;
      if (isA && bk == jb) {
        const double sd = sqrt(d), inv = 1.0 / sd;
#pragma unroll
        for (int ii = 0; ii < 8; ++ii) {
          const int i = 8 * bi + ii;
          const double l = (i > j) ? r[ii][jj] * inv : 0.0;
          if (i > j) r[ii][jj] = l;
          if (i == j) r[ii][jj] = sd;
          col[i] = l;
        }
        if (bi == jb && !(d > 0.0)) bad = j;
      } else if (!isA && bi == jb) {
        const double inv = 1.0 / sqrt(d);
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) {
          const double x = (bk <= jb) ? r[jj][cc] * inv : 0.0;
          if (bk <= jb) r[jj][cc] = x;
          xrow[8 * bk + cc] = x;
        }
      }
      __syncthreads();
      if (bad >= 0) break;
      // ---- trailing updates: a_ik -= l_ij l_kj ; b_ic -= l_ij x_jc
      double ci[8], ck[8];
#pragma unroll
      for (int ii = 0; ii < 8; ++ii) ci[ii] = col[8 * bi + ii];
      const double* src = isA ? col : xrow;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) ck[kk] = src[8 * bk + kk];
#pragma unroll
      for (int ii = 0; ii < 8; ++ii)
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) r[ii][kk] = fma(-ci[ii], ck[kk], r[ii][kk]);
      // next pivot (its owner updated it just above)
      if (isA && j + 1 < NB) {
        if (jj < 7) {
          if (bi == jb && bk == jb) piv = r[jj + 1][jj + 1];
        } else {
          if (bi == jb + 1 && bk == jb + 1) piv = r[0][0];
        }
      }
      __syncthreads();
    }
    if (bad >= 0) break;
  }
  if (bad >= 0) {
    if (tid == 0) {
      // reversed position p*NB + bad is processing index n - 1 - that
      const int64_t pos = (int64_t)p * NB + bad;
      *w.info = (pos < n) ? (long long)(n - 1 - pos) : (long long)-2;
      *w.flag = 1;
    }
    return;
  }
  if (!isA) {
#pragma unroll
    for (int ii = 0; ii < 8; ++ii)
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        w.Linv[(8 * bi + ii) * NB + 8 * bk + kk] =
            (act && (bi > bk || kk <= ii)) ? (float)r[ii][kk] : 0.f;
  }
}

// ------------------------------------------------------- tile products

// Layout of a global operand tile: element (x, k) of an X x K operand.
//   XK: stored row-major as [x][k] (leading dimension ld)
//   KX: stored row-major as [k][x]
enum { XK = 0, KX = 1 };

// Stage KS values of k for X consecutive x into LDS as sT[k][x] (stride LDT).
template <int LAY, int X>
__device__ inline void stage_load(float* sT, const float* G, int64_t ld, int k0) {
  const int tid = threadIdx.x;
  if (LAY == XK) {
#pragma unroll
    for (int q = 0; q < (X * KS / 4) / 256; ++q) {
      const int idx = tid + 256 * q;
      const int x = idx >> 3, k4 = (idx & 7) * 4;
      const float4 v = *reinterpret_cast<const float4*>(G + (int64_t)x * ld + k0 + k4);
      sT[(k4 + 0) * LDT + x] = v.x;
      sT[(k4 + 1) * LDT + x] = v.y;
      sT[(k4 + 2) * LDT + x] = v.z;
      sT[(k4 + 3) * LDT + x] = v.w;
    }
  } else {
#pragma unroll
    for (int q = 0; q < (X * KS / 4) / 256; ++q) {
      const int idx = tid + 256 * q;
      const int k = idx / (X / 4), x4 = (idx % (X / 4)) * 4;
      const float4 v = *reinterpret_cast<const float4*>(G + (int64_t)(k0 + k) * ld + x4);
      sT[k * LDT + x4 + 0] = v.x;
      sT[k * LDT + x4 + 1] = v.y;
      sT[k * LDT + x4 + 2] = v.z;
      sT[k * LDT + x4 + 3] = v.w;
    }
  }
}

// Workgroup tile product: out(x=i, y=j) = sum_k A(i, k) B(j, k) for an
// MR x MC output (MR = WR * TR * 32 rows, MC = WC * TC * 32 columns; four
// waves as WR x WC, each TR x TC accumulators of 32 x 32), K = NB.
template <int WR, int WC, int TR, int TC>
struct TileMma {
  static constexpr int MR = WR * TR * 32, MC = WC * TC * 32;
  f32x16_t acc[TR][TC];

  __device__ void zero() {
#pragma unroll
    for (int a = 0; a < TR; ++a)
#pragma unroll
      for (int b = 0; b < TC; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;
  }

  template <int LA, int LB>
  __device__ void run(const float* Ag, int64_t lda, const float* Bg, int64_t ldb, float* sA,
                      float* sB) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / WC, wn = wave % WC;
    const int lr = lane & 31, lk = lane >> 5;
    for (int k0 = 0; k0 < NB; k0 += KS) {
      __syncthreads();
      stage_load<LA, MR>(sA, Ag, lda, k0);
      stage_load<LB, MC>(sB, Bg, ldb, k0);
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < KS; kk += 2) {
        float af[TR], bf[TC];
#pragma unroll
        for (int a = 0; a < TR; ++a) af[a] = sA[(kk + lk) * LDT + (wm * TR + a) * 32 + lr];
#pragma unroll
        for (int b = 0; b < TC; ++b) bf[b] = sB[(kk + lk) * LDT + (wn * TC + b) * 32 + lr];
#pragma unroll
        for (int a = 0; a < TR; ++a)
#pragma unroll
          for (int b = 0; b < TC; ++b)
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[a], bf[b], acc[a][b], 0, 0, 0);
      }
    }
  }

  // MODE 0: C = acc; MODE 1: C -= acc.  32x32 accumulator layout: lane holds
  // column lane % 32; register v holds row 8 * (v / 4) + 4 * (lane / 32) + v % 4.
  template <int MODE>
  __device__ void store(float* C, int64_t ldc) const {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / WC, wn = wave % WC;
    const int lr = lane & 31, lk = lane >> 5;
#pragma unroll
    for (int a = 0; a < TR; ++a)
#pragma unroll
      for (int b = 0; b < TC; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = (wm * TR + a) * 32 + 8 * (v >> 2) + 4 * lk + (v & 3);
          const int c = (wn * TC + b) * 32 + lr;
          float* dst = C + (int64_t)r * ldc + c;
          if (MODE == 0) *dst = acc[a][b][v];
          else *dst -= acc[a][b][v];
        }
  }
};

// Quarter tiles (128 x 32) of Lp_i = A_ip Linv^T (i > p) and
// Yp_c = Linv B_pc (c <= p).
__global__ void __launch_bounds__(256) chol_panel(int64_t npad, int P, int p, CholWs w) {
  if (*w.flag) return;
  extern __shared__ __align__(16) float sm[];
  float* sA = sm;
  float* sB = sm + KS * LDT;
  const int q = P - p - 1;
  const int t = blockIdx.x >> 2, quarter = blockIdx.x & 3;
  TileMma<4, 1, 1, 1> mm;
  mm.zero();
  if (t < q) {
    const int i = p + 1 + t;
    const float* Aip = w.A + (int64_t)i * NB * npad + (int64_t)p * NB;
    // B(j, k) = Linv[32 quarter + j][k]
    mm.run<XK, XK>(Aip, npad, w.Linv + (int64_t)32 * quarter * NB, NB, sA, sB);
    mm.store<0>(w.Lp + (int64_t)i * NB * NB + 32 * quarter, NB);
  } else {
    const int c = t - q;
    // A(i, k) = Linv[i][k]; B(j, k) = B[p NB + k][c NB + 32 quarter + j]
    const float* Bpc = w.B + (int64_t)p * NB * npad + (int64_t)c * NB + 32 * quarter;
    mm.run<XK, KX>(w.Linv, NB, Bpc, npad, sA, sB);
    mm.store<0>(w.Yp + (int64_t)c * NB + 32 * quarter, npad);
  }
}

// SYRK tiles (i >= j > p), then forward-substitution tiles (i > p, c <= p),
// then the copy of Y_p into row block p of B.
__global__ void __launch_bounds__(256) chol_update(int64_t npad, int P, int p, CholWs w) {
  if (*w.flag) return;
  extern __shared__ __align__(16) float sm[];
  float* sA = sm;
  float* sB = sm + KS * LDT;
  const int q = P - p - 1;
  const int nsyrk = q * (q + 1) / 2;
  const int nfwd = q * (p + 1);
  int t = blockIdx.x;
  if (t < nsyrk + nfwd) {
    TileMma<2, 2, 2, 2> mm;
    mm.zero();
    if (t < nsyrk) {
      int a = 0;
      while (t >= a + 1) { t -= a + 1; ++a; }
      const int i = p + 1 + a, j = p + 1 + t;   // j <= i
      mm.run<XK, XK>(w.Lp + (int64_t)i * NB * NB, NB, w.Lp + (int64_t)j * NB * NB, NB, sA, sB);
      mm.store<1>(w.A + (int64_t)i * NB * npad + (int64_t)j * NB, npad);
    } else {
      t -= nsyrk;
      const int i = p + 1 + t / (p + 1), c = t % (p + 1);
      mm.run<XK, KX>(w.Lp + (int64_t)i * NB * NB, NB, w.Yp + (int64_t)c * NB, npad, sA, sB);
      mm.store<1>(w.B + (int64_t)i * NB * npad + (int64_t)c * NB, npad);
    }
  } else {
    const int c = t - nsyrk - nfwd;   // copy tile c of Y_p
    const float* src = w.Yp + (int64_t)c * NB;
    float* dst = w.B + (int64_t)p * NB * npad + (int64_t)c * NB;
    for (int e = threadIdx.x; e < NB * NB / 4; e += 256) {
      const int r = e / (NB / 4), c4 = (e % (NB / 4)) * 4;
      *reinterpret_cast<float4*>(dst + (int64_t)r * npad + c4) =
          *reinterpret_cast<const float4*>(src + (int64_t)r * npad + c4);
    }
  }
}

// R[a][b] = Y[n-1-a][n-1-b] for b >= a, 0 below the diagonal.
__global__ void __launch_bounds__(256) chol_flip(int64_t n, int64_t npad, float* R, int64_t ldr,
                                                 CholWs w) {
  if (*w.flag) return;
  const int64_t a = blockIdx.y;
  for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < n; b += (int64_t)gridDim.x * 256)
    R[a * ldr + b] = (b >= a) ? w.B[(n - 1 - a) * npad + (n - 1 - b)] : 0.f;
}

}  // namespace

size_t chol_ws_bytes(int64_t n) { return ws_layout(n, nullptr, nullptr); }

kronq_status chol_launch(const float* H, int64_t n, int64_t ldh, float lambda, int act_order,
                         int32_t* perm, float* R, int64_t ldr, int64_t* info, void* ws,
                         size_t ws_bytes, hipStream_t s) {
  (void)ws_bytes;
  CholWs w{};
  ws_layout(n, &w, ws);
  const int64_t npad = (n + NB - 1) / NB * NB;
  const int P = (int)(npad / NB);
  hipLaunchKernelGGL(chol_prep, dim3(1), dim3(256), 0, s, H, n, ldh, lambda, w);
  KQ_LAUNCHED("chol_prep");
  if (act_order) {
    hipLaunchKernelGGL(chol_act_order, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, H, n, ldh, perm);
    KQ_LAUNCHED("chol_act_order");
  } else {
    hipLaunchKernelGGL(chol_identity_perm, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, n, perm);
    KQ_LAUNCHED("chol_identity_perm");
  }
  {
    const unsigned gx = (unsigned)std::min<int64_t>((npad + 255) / 256, 64);
    hipLaunchKernelGGL(chol_gather, dim3(gx, (unsigned)npad), dim3(256), 0, s, H, n, ldh,
                       (const int32_t*)perm, npad, w);
    KQ_LAUNCHED("chol_gather");
  }
  const size_t lds_tile = 2 * (size_t)KS * LDT * sizeof(float);
  for (int p = 0; p < P; ++p) {
    hipLaunchKernelGGL(chol_diag, dim3(1), dim3(512), 0, s, npad, n, p, w);
    KQ_LAUNCHED("chol_diag");
    const int q = P - p - 1;
    hipLaunchKernelGGL(chol_panel, dim3(4 * (q + p + 1)), dim3(256), lds_tile, s, npad, P, p, w);
    KQ_LAUNCHED("chol_panel");
    const int tiles = q * (q + 1) / 2 + q * (p + 1) + (p + 1);
    hipLaunchKernelGGL(chol_update, dim3(tiles), dim3(256), lds_tile, s, npad, P, p, w);
    KQ_LAUNCHED("chol_update");
  }
  {
    const unsigned gx = (unsigned)std::min<int64_t>((n + 255) / 256, 64);
    hipLaunchKernelGGL(chol_flip, dim3(gx, (unsigned)n), dim3(256), 0, s, n, npad, R, ldr, w);
    KQ_LAUNCHED("chol_flip");
  }
  long long h_info = -1;
  int h_flag = 0;
  KQ_HIP(hipMemcpyAsync(&h_info, w.info, sizeof(h_info), hipMemcpyDeviceToHost, s));
  KQ_HIP(hipMemcpyAsync(&h_flag, w.flag, sizeof(h_flag), hipMemcpyDeviceToHost, s));
  KQ_HIP(hipStreamSynchronize(s));
  if (h_flag) {
    *info = h_info;
    return fail(KRONQ_ENOTPD, "kronq_chol_inv: trailing block at processing index %lld is not "
                "positive definite", h_info);
  }
  *info = -1;
  return KRONQ_OK;
}

}  // namespace kronq
