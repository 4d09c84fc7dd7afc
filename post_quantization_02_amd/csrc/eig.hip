// Symmetric eigen-decomposition for the mu-incoherence diagnostic (hyper.ai
// summary of the KronQ paper, Method, and the Pith review's Figure 2(a): the
// incoherence of a proxy Hessian, mu(H)/sqrt(d) = max_ij |Q_ij| over the
// eigenvector matrix Q of H = Q Lambda Q^T).
//
// Two-sided block Jacobi in fp64.  The (padded) index set is cut into blocks
// of 16; a sweep pairs every two blocks once, in the rounds of a round-robin
// tournament (nb/2 disjoint pairs per round, nb - 1 rounds).  Per round:
//   eig_solve : one workgroup per pair diagonalizes the 32 x 32 submatrix of
//               its two blocks completely (cyclic Jacobi in LDS, parallel
//               ordering, 16 rotations at a time) and stores the orthogonal
//               32 x 32 factor Q_k and the diagonal it reached;
//   eig_apply : A <- J^T A J and V <- V J, with J the direct sum of the Q_k
//               over the round's pairs.  The tile of A at (pair r, pair c) is
//               Q_r^T A_rc Q_c, and the tiles partition A, so each workgroup
//               updates its tile (and the mirrored one) in place; a pair's own
//               tile becomes the diagonal the solver reached, with exact zeros
//               off it (as scalar Jacobi sets each annihilated entry to zero),
//               which keeps product rounding out of the converged part.  V's
//               tiles are 32 rows x one pair's columns.
// A sweep ends with the off-diagonal norm; the host stops when it is below
// tol times the Frobenius norm.  Padded indices have zero rows and columns,
// are never rotated (a zero coupling gives the identity rotation) and stay
// out of the results.
#include <cmath>

#include "kronq_internal.h"

namespace kronq {
namespace {

constexpr int EB = 16;          // block of indices
constexpr int EP = 2 * EB;      // a pair's submatrix order
constexpr int ENT = 256;        // threads per workgroup
constexpr int ELD = EP + 1;     // LDS row stride (doubles)
constexpr int kRedBlocks = 256;
constexpr int kInnerSweeps = 12;
constexpr double kInnerTol = 1e-14;

// pair k of round r of a round-robin tournament on `teams` (even) teams
__device__ __forceinline__ void rr_pair(int teams, int r, int k, int& a, int& b) {
  const int M = teams - 1;
  if (k == 0) {
    a = M;
    b = r;
  } else {
    a = (r + k) % M;
    b = (r - k + M) % M;
  }
}

__device__ __forceinline__ int64_t pair_index(int bi, int bj, int i) {
  return i < EB ? (int64_t)bi * EB + i : (int64_t)bj * EB + (i - EB);
}

// block sum of two doubles into out[0..1] (all threads get the result)
__device__ __forceinline__ void block_sum2(double& a, double& b, double* red) {
  for (int o = 32; o > 0; o >>= 1) {
    a += __shfl_xor(a, o);
    b += __shfl_xor(b, o);
  }
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  if (l == 0) {
    red[2 * w] = a;
    red[2 * w + 1] = b;
  }
  __syncthreads();
  a = 0.0;
  b = 0.0;
  for (int k = 0; k < ENT / 64; ++k) {
    a += red[2 * k];
    b += red[2 * k + 1];
  }
  __syncthreads();
}

__global__ void __launch_bounds__(ENT) eig_init(const float* __restrict__ H, int64_t n, int64_t ldh,
                                                int64_t npad, double* __restrict__ A,
                                                double* __restrict__ V) {
  const int64_t total = npad * npad;
  for (int64_t e = (int64_t)blockIdx.x * ENT + threadIdx.x; e < total; e += (int64_t)gridDim.x * ENT) {
    const int64_t i = e / npad, j = e % npad;
    double a = 0.0;
    if (i < n && j < n) a = (double)(i >= j ? H[i * ldh + j] : H[j * ldh + i]);   // lower triangle
    A[e] = a;
    V[e] = i == j ? 1.0 : 0.0;
  }
}

// Jacobi rotation (c, s) that zeroes S[p][q] of the 2 x 2 [[app, apq], [apq, aqq]]
// under J = [[c, s], [-s, c]] (J^T S J): t = tan(theta) is the smaller root of
// t^2 + 2 tau t - 1 = 0 with tau = (aqq - app) / (2 apq).
__device__ __forceinline__ void jacobi_rot(double app, double aqq, double apq, double& c, double& s) {
  if (apq == 0.0) {
    c = 1.0;
    s = 0.0;
    return;
  }
  const double tau = (aqq - app) / (2.0 * apq);
  const double t = (tau >= 0.0 ? 1.0 : -1.0) / (fabs(tau) + hypot(1.0, tau));
  c = 1.0 / sqrt(1.0 + t * t);
  s = t * c;
}

__global__ void __launch_bounds__(ENT) eig_solve(const double* __restrict__ A, int64_t npad, int nb,
                                                 int round, double* __restrict__ Qp,
                                                 double* __restrict__ Dp) {
  __shared__ double S[EP * ELD];
  __shared__ double Q[EP * ELD];
  __shared__ double cs[EB][2];
  __shared__ int pq[EB][2];
  __shared__ double red[2 * (ENT / 64)];
  const int k = blockIdx.x, tid = threadIdx.x;
  int bi, bj;
  rr_pair(nb, round, k, bi, bj);
  for (int e = tid; e < EP * EP; e += ENT) {
    const int i = e / EP, j = e % EP;
    S[i * ELD + j] = A[pair_index(bi, bj, i) * npad + pair_index(bi, bj, j)];
    Q[i * ELD + j] = i == j ? 1.0 : 0.0;
  }
  if (tid < EB) pq[tid][0] = pq[tid][1] = -1;
  __syncthreads();
  for (int sw = 0; sw < kInnerSweeps; ++sw) {
    double off = 0.0, tot = 0.0;
    for (int e = tid; e < EP * EP; e += ENT) {
      const int i = e / EP, j = e % EP;
      const double v = S[i * ELD + j];
      tot += v * v;
      if (i != j) off += v * v;
    }
    block_sum2(off, tot, red);
    if (off <= kInnerTol * kInnerTol * tot) break;
    for (int r = 0; r < EP - 1; ++r) {
      if (tid < EB) {
        // the previous round's rotated pair: its coupling is zero by construction
        if (pq[tid][0] >= 0 && cs[tid][1] != 0.0) {
          S[pq[tid][0] * ELD + pq[tid][1]] = 0.0;
          S[pq[tid][1] * ELD + pq[tid][0]] = 0.0;
        }
        int p, q;
        rr_pair(EP, r, tid, p, q);
        double c, s;
        jacobi_rot(S[p * ELD + p], S[q * ELD + q], S[p * ELD + q], c, s);
        cs[tid][0] = c;
        cs[tid][1] = s;
        pq[tid][0] = p;
        pq[tid][1] = q;
      }
      __syncthreads();
      // rows p, q <- J^T rows
      for (int e = tid; e < EB * EP; e += ENT) {
        const int t = e / EP, j = e % EP;
        const int p = pq[t][0], q = pq[t][1];
        const double c = cs[t][0], s = cs[t][1];
        const double sp = S[p * ELD + j], sq = S[q * ELD + j];
        S[p * ELD + j] = c * sp - s * sq;
        S[q * ELD + j] = s * sp + c * sq;
      }
      __syncthreads();
      // columns p, q of S and of Q <- columns J
      for (int e = tid; e < 2 * EB * EP; e += ENT) {
        double* M = e < EB * EP ? S : Q;
        const int f = e % (EB * EP);
        const int t = f / EP, i = f % EP;
        const int p = pq[t][0], q = pq[t][1];
        const double c = cs[t][0], s = cs[t][1];
        const double mp = M[i * ELD + p], mq = M[i * ELD + q];
        M[i * ELD + p] = c * mp - s * mq;
        M[i * ELD + q] = s * mp + c * mq;
      }
      __syncthreads();
    }
    if (tid < EB && pq[tid][0] >= 0 && cs[tid][1] != 0.0) {
      S[pq[tid][0] * ELD + pq[tid][1]] = 0.0;
      S[pq[tid][1] * ELD + pq[tid][0]] = 0.0;
    }
    if (tid < EB) pq[tid][0] = -1;
    __syncthreads();
  }
  double* out = Qp + (int64_t)k * EP * EP;
  for (int e = tid; e < EP * EP; e += ENT) out[e] = Q[(e / EP) * ELD + e % EP];
  if (tid < EP) Dp[(int64_t)k * EP + tid] = S[tid * ELD + tid];
}

// A <- J^T A J on the upper tiles (mirrored), V <- V J; blocks [0, np2*np2) are
// A tiles (row pair, column pair), the rest V tiles (32-row strip, column pair)
__global__ void __launch_bounds__(ENT) eig_apply(double* __restrict__ A, double* __restrict__ V,
                                                 int64_t npad, int nb, int round,
                                                 const double* __restrict__ Qp,
                                                 const double* __restrict__ Dp) {
  __shared__ double T[EP * ELD];
  __shared__ double U[EP * ELD];
  __shared__ double Qr[EP * ELD];
  __shared__ double Qc[EP * ELD];
  const int np2 = nb / 2;
  const int tid = threadIdx.x;
  const int64_t b = blockIdx.x;
  const int64_t nA = (int64_t)np2 * np2;
  const bool isA = b < nA;
  int kr, kc;
  if (isA) {
    kr = (int)(b / np2);
    kc = (int)(b % np2);
    if (kr > kc) return;
  } else {
    kr = (int)((b - nA) / np2);   // 32-row strip of V
    kc = (int)((b - nA) % np2);
  }
  int ri = 0, rj = 0, ci, cj;
  if (isA) rr_pair(nb, round, kr, ri, rj);
  rr_pair(nb, round, kc, ci, cj);
  if (isA && kr == kc) {
    // the pair's own tile: the solver's diagonal, zeros elsewhere
    for (int e = tid; e < EP * EP; e += ENT) {
      const int i = e / EP, j = e % EP;
      A[pair_index(ri, rj, i) * npad + pair_index(ci, cj, j)] = i == j ? Dp[(int64_t)kr * EP + i] : 0.0;
    }
    return;
  }
  const double* qc = Qp + (int64_t)kc * EP * EP;
  const double* qr = Qp + (int64_t)kr * EP * EP;
  for (int e = tid; e < EP * EP; e += ENT) {
    const int i = e / EP, j = e % EP;
    const int64_t gi = isA ? pair_index(ri, rj, i) : (int64_t)kr * EP + i;
    const int64_t gj = pair_index(ci, cj, j);
    T[i * ELD + j] = (isA ? A : V)[gi * npad + gj];
    Qc[i * ELD + j] = qc[e];
    if (isA) Qr[i * ELD + j] = qr[e];
  }
  __syncthreads();
  // U = T Q_c
  for (int e = tid; e < EP * EP; e += ENT) {
    const int i = e / EP, j = e % EP;
    double acc = 0.0;
#pragma unroll 8
    for (int l = 0; l < EP; ++l) acc += T[i * ELD + l] * Qc[l * ELD + j];
    U[i * ELD + j] = acc;
  }
  __syncthreads();
  if (!isA) {
    for (int e = tid; e < EP * EP; e += ENT) {
      const int i = e / EP, j = e % EP;
      V[((int64_t)kr * EP + i) * npad + pair_index(ci, cj, j)] = U[i * ELD + j];
    }
    return;
  }
  // T = Q_r^T U
  for (int e = tid; e < EP * EP; e += ENT) {
    const int i = e / EP, j = e % EP;
    double acc = 0.0;
#pragma unroll 8
    for (int l = 0; l < EP; ++l) acc += Qr[l * ELD + i] * U[l * ELD + j];
    T[i * ELD + j] = acc;
  }
  __syncthreads();
  for (int e = tid; e < EP * EP; e += ENT) {
    const int i = e / EP, j = e % EP;
    A[pair_index(ri, rj, i) * npad + pair_index(ci, cj, j)] = T[i * ELD + j];
    // the mirrored tile, written row by row (coalesced over j)
    A[pair_index(ci, cj, i) * npad + pair_index(ri, rj, j)] = T[j * ELD + i];
  }
}

// per-block sums of the squared off-diagonal and of all squared entries
__global__ void __launch_bounds__(ENT) eig_offnorm(const double* __restrict__ A, int64_t npad,
                                                   double* __restrict__ part) {
  __shared__ double red[2 * (ENT / 64)];
  double off = 0.0, tot = 0.0;
  const int64_t total = npad * npad;
  for (int64_t e = (int64_t)blockIdx.x * ENT + threadIdx.x; e < total; e += (int64_t)gridDim.x * ENT) {
    const double v = A[e];
    tot += v * v;
    if (e / npad != e % npad) off += v * v;
  }
  block_sum2(off, tot, red);
  if (threadIdx.x == 0) {
    part[2 * blockIdx.x] = off;
    part[2 * blockIdx.x + 1] = tot;
  }
}

__global__ void __launch_bounds__(ENT) eig_sum_parts(const double* __restrict__ part, int nparts,
                                                     double* __restrict__ out) {
  __shared__ double red[2 * (ENT / 64)];
  double a = 0.0, b = 0.0;
  for (int k = threadIdx.x; k < nparts; k += ENT) {
    a += part[2 * k];
    b += part[2 * k + 1];
  }
  block_sum2(a, b, red);
  if (threadIdx.x == 0) {
    out[0] = a;
    out[1] = b;
  }
}

// eigenvalues, eigenvectors (n x n of V) and per-block max |V_ij|, i, j < n
__global__ void __launch_bounds__(ENT) eig_finish(const double* __restrict__ A,
                                                  const double* __restrict__ V, int64_t npad,
                                                  int64_t n, double* __restrict__ evals,
                                                  double* __restrict__ Q, int64_t ldq,
                                                  double* __restrict__ part) {
  __shared__ double red[ENT / 64];
  double mx = 0.0;
  const int64_t total = n * n;
  for (int64_t e = (int64_t)blockIdx.x * ENT + threadIdx.x; e < total; e += (int64_t)gridDim.x * ENT) {
    const int64_t i = e / n, j = e % n;
    const double v = V[i * npad + j];
    mx = fmax(mx, fabs(v));
    if (Q) Q[i * ldq + j] = v;
    if (evals && i == j) evals[i] = A[i * npad + i];
  }
  for (int o = 32; o > 0; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < ENT / 64; ++k) mx = fmax(mx, red[k]);
    part[blockIdx.x] = fmax(mx, red[0]);
  }
}

__global__ void __launch_bounds__(ENT) eig_max_parts(const double* __restrict__ part, int nparts,
                                                     double* __restrict__ out) {
  __shared__ double red[ENT / 64];
  double mx = 0.0;
  for (int k = threadIdx.x; k < nparts; k += ENT) mx = fmax(mx, part[k]);
  for (int o = 32; o > 0; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < ENT / 64; ++k) mx = fmax(mx, red[k]);
    out[0] = fmax(mx, red[0]);
  }
}

int64_t eig_npad(int64_t n) { return (n + EP - 1) / EP * EP; }

struct EigWs {
  double *A, *V, *Qp, *Dp, *part, *out;
};

EigWs eig_carve(void* ws, int64_t n) {
  const int64_t npad = eig_npad(n);
  const size_t mat = align_up((size_t)npad * npad * sizeof(double), 256);
  const size_t qp = align_up((size_t)(npad / EP) * EP * EP * sizeof(double), 256);
  const size_t part = align_up((size_t)2 * kRedBlocks * sizeof(double), 256);
  char* p = static_cast<char*>(ws);
  EigWs w;
  w.A = reinterpret_cast<double*>(p);
  w.V = reinterpret_cast<double*>(p + mat);
  w.Qp = reinterpret_cast<double*>(p + 2 * mat);
  const size_t dp = align_up((size_t)npad * sizeof(double), 256);
  w.Dp = reinterpret_cast<double*>(p + 2 * mat + qp);
  w.part = reinterpret_cast<double*>(p + 2 * mat + qp + dp);
  w.out = reinterpret_cast<double*>(p + 2 * mat + qp + dp + part);
  return w;
}

}  // namespace

size_t eig_ws_bytes(int64_t n) {
  const int64_t npad = eig_npad(n);
  return 2 * align_up((size_t)npad * npad * sizeof(double), 256) +
         align_up((size_t)(npad / EP) * EP * EP * sizeof(double), 256) +
         align_up((size_t)npad * sizeof(double), 256) +
         align_up((size_t)2 * kRedBlocks * sizeof(double), 256) + 256;
}

kronq_status eig_launch(const float* H, int64_t n, int64_t ldh, double tol, int max_sweeps,
                        double* mu, double* evals, double* Q, int64_t ldq, int32_t* sweeps, void* ws,
                        hipStream_t s) {
  const int64_t npad = eig_npad(n);
  const int nb = (int)(npad / EB);   // even
  const EigWs w = eig_carve(ws, n);
  const int64_t tot = npad * npad;
  const unsigned gfill = (unsigned)std::min<int64_t>((tot + ENT - 1) / ENT, 8192);
  hipLaunchKernelGGL(eig_init, dim3(gfill), dim3(ENT), 0, s, H, n, ldh, npad, w.A, w.V);
  KQ_LAUNCHED("eig_init");
  const unsigned gred = (unsigned)std::min<int64_t>((tot + ENT - 1) / ENT, kRedBlocks);
  const int np2 = nb / 2;
  const unsigned gapply = (unsigned)((int64_t)np2 * np2 + (npad / EP) * np2);
  int sw = 0;
  bool converged = false;
  for (;; ++sw) {
    hipLaunchKernelGGL(eig_offnorm, dim3(gred), dim3(ENT), 0, s, w.A, npad, w.part);
    KQ_LAUNCHED("eig_offnorm");
    hipLaunchKernelGGL(eig_sum_parts, dim3(1), dim3(ENT), 0, s, w.part, (int)gred, w.out);
    KQ_LAUNCHED("eig_sum_parts");
    double h[2];
    KQ_HIP(hipMemcpyAsync(h, w.out, sizeof(h), hipMemcpyDeviceToHost, s));
    KQ_HIP(hipStreamSynchronize(s));
    if (!std::isfinite(h[0]) || !std::isfinite(h[1]))
      return fail(KRONQ_ENUMERIC, "kronq_incoherence: H holds a NaN or an infinity");
    if (h[0] <= tol * tol * h[1]) {
      converged = true;
      break;
    }
    if (sw >= max_sweeps) break;
    for (int r = 0; r < nb - 1; ++r) {
      hipLaunchKernelGGL(eig_solve, dim3((unsigned)np2), dim3(ENT), 0, s, w.A, npad, nb, r, w.Qp, w.Dp);
      KQ_LAUNCHED("eig_solve");
      hipLaunchKernelGGL(eig_apply, dim3(gapply), dim3(ENT), 0, s, w.A, w.V, npad, nb, r, w.Qp, w.Dp);
      KQ_LAUNCHED("eig_apply");
    }
  }
  if (sweeps) *sweeps = sw;
  if (!converged)
    return fail(KRONQ_ENUMERIC, "kronq_incoherence: no convergence to %g in %d sweeps", tol, max_sweeps);
  const unsigned gfin = (unsigned)std::min<int64_t>((n * n + ENT - 1) / ENT, kRedBlocks);
  hipLaunchKernelGGL(eig_finish, dim3(gfin), dim3(ENT), 0, s, w.A, w.V, npad, n, evals, Q, ldq, w.part);
  KQ_LAUNCHED("eig_finish");
  hipLaunchKernelGGL(eig_max_parts, dim3(1), dim3(ENT), 0, s, w.part, (int)gfin, w.out);
  KQ_LAUNCHED("eig_max_parts");
  KQ_HIP(hipMemcpyAsync(mu, w.out, sizeof(double), hipMemcpyDeviceToHost, s));
  KQ_HIP(hipStreamSynchronize(s));
  return KRONQ_OK;
}

}  // namespace kronq
