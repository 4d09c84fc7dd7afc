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
//   diag kernel   (1 workgroup): Cholesky of A_pp and Linv_pp in fp64, blocked
//                 by 32 columns (one wave factors and inverts each 32 x 32
//                 diagonal sub-block in registers; the sub-block products run
//                 on the fp64 matrix cores); pivots <= 0 are reported
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
//
// Factor the diagonal block S = A_pp = L L^T and invert L (fp64, one
// workgroup of four waves), blocked by SB = 32 columns:
//   for kb = 0..3:
//     B1 (wave 0): S_kk = L_kk L_kk^T and M_kk = L_kk^-1 column by column in
//        registers: lanes 0..31 hold the rows of S_kk, lanes 32..63 the
//        columns of the identity that becomes M_kk.  At step j both halves
//        apply v[k] -= (v[j] / d) c[k] for k > j, with c = column j of S_kk
//        (passed through LDS) and d = c[j]; the M half then scales v[j] by
//        1 / sqrt(d).  No barrier inside.
//     B2: L_ik = S_ik M_kk^T           (kb < i, one wave per block)
//     B3: S_ij -= L_ik L_jk^T           (kb < j <= i)
//   C: the blocked triangular inverse, one row block at a time:
//      X_ii = M_ii,  X_ij = -M_ii sum_{k=j}^{i-1} L_ik X_kj   (j < i)
// Only the lower triangle of S is read.  Block products are 32 x 32 x 32 on
// v_mfma_f64_16x16x4f64, one wave each.

constexpr int SB = 32;
constexpr int NSB = NB / SB;       // sub-blocks per side
constexpr int LDB = SB + 1;        // LDS row stride of a stored sub-block (doubles)
constexpr int BLKD = SB * LDB;     // doubles per stored sub-block

typedef double f64x4_t __attribute__((__vector_size__(4 * sizeof(double))));

// lower sub-block (i >= j) -> slot
__device__ __forceinline__ int lslot(int i, int j) { return i * (i + 1) / 2 + j; }

// acc (2 x 2 tiles of 16 x 16) += sign * A B over 32 k, A(r, t) = pa[r * sar + t * sat],
// B(t, c) = pb[t * sbt + c * sbc] (LDS).  Lane l supplies A(16 ti + l % 16, k0 + l / 16)
// and B(k0 + l / 16, 16 tj + l % 16); register v of tile (ti, tj) holds element
// (16 ti + 4 v + l / 16, 16 tj + l % 16).
__device__ __forceinline__ void bmma(f64x4_t (&acc)[2][2], const double* pa, int sar, int sat,
                                     const double* pb, int sbt, int sbc, double sign) {
  const int l = threadIdx.x & 63, r = l & 15, kk = l >> 4;
#pragma unroll
  for (int k0 = 0; k0 < SB; k0 += 4) {
    double av[2], bv[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      av[t] = sign * pa[(16 * t + r) * sar + (k0 + kk) * sat];
      bv[t] = pb[(k0 + kk) * sbt + (16 * t + r) * sbc];
    }
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int tj = 0; tj < 2; ++tj)
        acc[ti][tj] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[ti], bv[tj], acc[ti][tj], 0, 0, 0);
  }
}

__device__ __forceinline__ void bzero(f64x4_t (&acc)[2][2]) {
#pragma unroll
  for (int ti = 0; ti < 2; ++ti)
#pragma unroll
    for (int tj = 0; tj < 2; ++tj) acc[ti][tj] = f64x4_t{0.0, 0.0, 0.0, 0.0};
}

__device__ __forceinline__ void bload(f64x4_t (&acc)[2][2], const double* blk) {
  const int l = threadIdx.x & 63;
#pragma unroll
  for (int ti = 0; ti < 2; ++ti)
#pragma unroll
    for (int tj = 0; tj < 2; ++tj)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[ti][tj][v] = blk[(16 * ti + 4 * v + (l >> 4)) * LDB + 16 * tj + (l & 15)];
}

__device__ __forceinline__ void bstore(const f64x4_t (&acc)[2][2], double* blk) {
  const int l = threadIdx.x & 63;
#pragma unroll
  for (int ti = 0; ti < 2; ++ti)
#pragma unroll
    for (int tj = 0; tj < 2; ++tj)
#pragma unroll
      for (int v = 0; v < 4; ++v) blk[(16 * ti + 4 * v + (l >> 4)) * LDB + 16 * tj + (l & 15)] = acc[ti][tj][v];
}

// B1 on one wave: factor the stored block Sk (lower triangle read) and write
// M = L^-1 (lower triangular) to Mk.  Returns the first column whose pivot is
// not positive (or NaN), else -1; past a failed pivot the sweep continues with
// d = 1 and its results are discarded.
__device__ __noinline__ int diag_factor32(const double* Sk, double* Mk, double* col) {
  const int l = threadIdx.x & 63, r = l & 31;
  const bool isS = l < 32;
  double v[SB], c[SB];
#pragma unroll
  for (int k = 0; k < SB; ++k) v[k] = isS ? Sk[max(r, k) * LDB + min(r, k)] : (k == r ? 1.0 : 0.0);
  if (isS) col[r] = v[0];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int k = 0; k < SB; ++k) c[k] = col[k];
  int bad = -1;
#pragma unroll
  for (int j = 0; j < SB; ++j) {
    double d = c[j];
    if (!(d > 0.0)) {
      if (bad < 0) bad = j;
      d = 1.0;
    }
    // y = 1 / sqrt(d): hardware estimate refined by two Newton-Raphson steps
    // y <- y (3 - d y^2) / 2
    double y = __builtin_amdgcn_rsq(d);
    y = y * fma(-0.5 * d, y * y, 1.5);
    y = y * fma(-0.5 * d, y * y, 1.5);
    const double coef = v[j] * (y * y);
    double cn[SB];
    if (j + 1 < SB) {
      // next column first, so that its broadcast overlaps the rest of the update
      v[j + 1] = fma(-coef, c[j + 1], v[j + 1]);
      if (isS) col[r] = v[j + 1];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int k = 0; k < SB; ++k) cn[k] = col[k];
    }
#pragma unroll
    for (int k = j + 2; k < SB; ++k) v[k] = fma(-coef, c[k], v[k]);
    if (!isS) v[j] *= y;
    if (j + 1 < SB) {
#pragma unroll
      for (int k = 0; k < SB; ++k) c[k] = cn[k];
    }
  }
  if (!isS) {
#pragma unroll
    for (int i = 0; i < SB; ++i) Mk[i * LDB + r] = v[i];
  }
  return bad;
}

__global__ void __launch_bounds__(256) chol_diag(int64_t npad, int64_t n, int p, CholWs w) {
  if (*w.flag) return;
  __shared__ double Ls[NSB * (NSB + 1) / 2 * BLKD];  // lower sub-blocks of S, then L, then X
  __shared__ double Ms[NSB * BLKD];                  // M_kk = L_kk^-1
  __shared__ double Ts[(NSB - 1) * BLKD];            // per-wave scratch of the inverse
  __shared__ __align__(16) double col[SB];
  __shared__ int s_bad;
  const int tid = threadIdx.x, wave = tid >> 6;

  // ---- A: load the lower sub-blocks of A_pp (fp32 -> fp64)
  {
    const float* Ap = w.A + (int64_t)p * NB * npad + (int64_t)p * NB;
    constexpr int NQ = NSB * (NSB + 1) / 2 * SB * (SB / 4);  // float4 count
    for (int e = tid; e < NQ; e += 256) {
      const int blk = e / (SB * SB / 4), rem = e % (SB * SB / 4);
      const int r = rem / (SB / 4), c4 = (rem % (SB / 4)) * 4;
      int bi = 0;
      while (lslot(bi + 1, 0) <= blk) ++bi;
      const int bj = blk - lslot(bi, 0);
      const float4 v = *reinterpret_cast<const float4*>(Ap + (int64_t)(SB * bi + r) * npad + SB * bj + c4);
      double* dst = Ls + blk * BLKD + r * LDB + c4;
      dst[0] = v.x;
      dst[1] = v.y;
      dst[2] = v.z;
      dst[3] = v.w;
    }
  }
  if (tid == 0) s_bad = -1;
  __syncthreads();

  // ---- B: blocked factorization
  for (int kb = 0; kb < NSB; ++kb) {
    if (wave == 0) {
      const int bad = diag_factor32(Ls + lslot(kb, kb) * BLKD, Ms + kb * BLKD, col);
      if (tid == 0 && bad >= 0) s_bad = SB * kb + bad;
    }
    __syncthreads();
    if (s_bad >= 0) break;
    // B2: L_ik = S_ik M_kk^T
    {
      const int i = kb + 1 + wave;
      if (i < NSB) {
        f64x4_t acc[2][2];
        bzero(acc);
        double* Sik = Ls + lslot(i, kb) * BLKD;
        bmma(acc, Sik, LDB, 1, Ms + kb * BLKD, 1, LDB, 1.0);
        bstore(acc, Sik);
      }
    }
    __syncthreads();
    // B3: S_ij -= L_ik L_jk^T for kb < j <= i
    {
      const int q = NSB - 1 - kb;  // trailing sub-blocks per side
      for (int t = wave; t < q * (q + 1) / 2; t += 4) {
        int a = 0, u = t;
        while (u > a) { u -= a + 1; ++a; }
        const int i = kb + 1 + a, j = kb + 1 + u;
        f64x4_t acc[2][2];
        double* Sij = Ls + lslot(i, j) * BLKD;
        bload(acc, Sij);
        bmma(acc, Ls + lslot(i, kb) * BLKD, LDB, 1, Ls + lslot(j, kb) * BLKD, 1, LDB, -1.0);
        bstore(acc, Sij);
      }
    }
    __syncthreads();
  }
  if (s_bad >= 0) {
    if (tid == 0) {
      // reversed position p*NB + bad is processing index n - 1 - that
      const int64_t pos = (int64_t)p * NB + s_bad;
      *w.info = (pos < n) ? (long long)(n - 1 - pos) : (long long)-2;
      *w.flag = 1;
    }
    return;
  }

  // ---- C: X = L^-1, row block by row block (X_ij overwrites L_ij)
  for (int i = 1; i < NSB; ++i) {
    f64x4_t x[2][2];
    if (wave < i) {
      const int j = wave;
      f64x4_t acc[2][2];
      bzero(acc);
      for (int k = j; k < i; ++k) {
        const double* Xkj = (k == j) ? Ms + j * BLKD : Ls + lslot(k, j) * BLKD;
        bmma(acc, Ls + lslot(i, k) * BLKD, LDB, 1, Xkj, LDB, 1, 1.0);
      }
      bstore(acc, Ts + j * BLKD);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      bzero(x);
      bmma(x, Ms + i * BLKD, LDB, 1, Ts + j * BLKD, LDB, 1, -1.0);
    }
    __syncthreads();
    if (wave < i) bstore(x, Ls + lslot(i, wave) * BLKD);
    __syncthreads();
  }

  // ---- D: Linv (fp32, NB x NB, zeros above the diagonal)
  for (int e = tid; e < NB * NB; e += 256) {
    const int r = e / NB, c = e % NB;
    const int bi = r / SB, bj = c / SB, rr = r % SB, cc = c % SB;
    float v = 0.f;
    if (bi > bj) v = (float)Ls[lslot(bi, bj) * BLKD + rr * LDB + cc];
    else if (bi == bj) v = (float)Ms[bi * BLKD + rr * LDB + cc];
    w.Linv[e] = v;
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
    hipLaunchKernelGGL(chol_diag, dim3(1), dim3(256), 0, s, npad, n, p, w);
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
