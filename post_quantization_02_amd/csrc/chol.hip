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
//   panel kernels : PL: Lp_i = A_ip Linv_pp^T (i > p) and PY: Yp_c = Linv_pp
//                   B_pc (c <= p), each as four 128 x 32 quarter tiles
//   update kernels: U1: A_i,p+1 -= Lp_i Lp_p+1^T (i > p; the next column),
//                   U2: A_ij -= Lp_i Lp_j^T (i >= j > p + 1; Cholesky SYRK),
//                       B_ic -= Lp_i Yp_c   (i > p, c <= p; forward
//                       substitution), B_pc = Yp_c (row block p of Y = L^-1)
// and finally R = J Y J.  Tile products run on the fp32 matrix cores
// (v_mfma_f32_32x32x2f32).
//
// Look-ahead in one stream: U2(p - 1) runs in the same launch as diag(p)
// (workgroup 0 takes the diagonal block, the others the U2 tiles), then PL(p)
// and PY(p) share a launch, then U1(p).  The critical path diag(p) -> PL(p) ->
// U1(p) -> diag(p + 1) so never waits on the large update, and no event
// crosses streams.  U2(p - 1) writes columns past p and row blocks of B past
// p - 1, so it is independent of diag(p); U1(p) writes column p + 1 after
// U2(p - 1), which also writes it, has finished.  Linv, Lp and Yp are
// double-buffered by the parity of p (diag(p) writes Linv of parity p while
// U2(p - 1) reads Lp and Yp of the other).  A device flag set by a failed
// pivot makes every later kernel return at once; the host reads the flag
// after the last launch.

#include "kronq_internal.h"

namespace kronq {
namespace {

typedef float f32x16_t __attribute__((__vector_size__(16 * sizeof(float))));

constexpr int NB = 128;
constexpr int KS = 32;        // K rows per LDS stage
constexpr int NBO = 4;        // panels of an outer block (two-level sweep)
constexpr int kTwoLevelMinPanels = 64;   // two-level from n > 8064 on (measured crossover)

struct CholWs {
  float* A;       // npad x npad (reversed, permuted, damped)
  float* B;       // npad x npad (forward substitution; ends as Y = L^-1)
  float* Lp;      // npad x NB   (panel L_ip of step p; two buffers by p % 2)
  float* Yp;      // NB x npad   (row block Y_p of step p; two buffers)
  float* Linv;    // NB x NB     (inverse of diagonal block p; two buffers)
  double* damp;   // lambda * mean(diag H)
  int* flag;      // nonzero after a failed pivot or a non-finite input
  int* nonfinite; // nonzero when H (or the damping term) holds a NaN or infinity
  long long* info;
  int64_t sP;     // floats between consecutive Lp (and Yp) buffers (NBO of each)
  unsigned short* Ls;  // two-level sweep: the bf16 parts of the outer block's L
                       // panels, k-major: [slot][k / 32][part][k % 32][row]
  unsigned short* Ys;  // and of its Y panels: [slot][k / 32][part][k % 32][column]
};

// buffer of parity `par` of a double-buffered array
__device__ __forceinline__ float* lp_buf(const CholWs& w, int par) { return w.Lp + par * w.sP; }
__device__ __forceinline__ float* yp_buf(const CholWs& w, int par) { return w.Yp + par * w.sP; }
__device__ __forceinline__ float* linv_buf(const CholWs& w, int par) { return w.Linv + par * NB * NB; }

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
  off += NBO * sP;
  if (w) w->Yp = reinterpret_cast<float*>(b + off);
  off += NBO * sP;
  if (w) w->Linv = reinterpret_cast<float*>(b + off);
  off += 2 * align_up((size_t)NB * NB * sizeof(float), 256);
  if (w) w->sP = (int64_t)(sP / sizeof(float));
  if (w) w->damp = reinterpret_cast<double*>(b + off);
  off += 256;
  if (w) w->flag = reinterpret_cast<int*>(b + off);
  off += 256;
  if (w) w->info = reinterpret_cast<long long*>(b + off);
  off += 256;
  if (w) w->nonfinite = reinterpret_cast<int*>(b + off);
  off += 256;
  if (npad / NB >= kTwoLevelMinPanels) {
    const size_t sS = align_up((size_t)NBO * 3 * npad * NB * sizeof(unsigned short), 256);
    if (w) w->Ls = reinterpret_cast<unsigned short*>(b + off);
    off += sS;
    if (w) w->Ys = reinterpret_cast<unsigned short*>(b + off);
    off += sS;
  }
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
    *w.nonfinite = 0;
    *w.info = -1;
  }
}

// an fp32 value is NaN or infinite exactly when its exponent field is all ones
__device__ __forceinline__ bool nonfinite_bits(float v) {
  return (__float_as_uint(v) & 0x7f800000u) == 0x7f800000u;
}

// a non-finite entry of the damped matrix stops the factorization: every
// later kernel sees the flag and returns
__device__ __forceinline__ void mark_nonfinite(const CholWs& w) {
  *w.nonfinite = 1;
  *w.flag = 1;
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
      if (nonfinite_bits(v)) mark_nonfinite(w);
    } else {
      v = (a == b) ? 1.f : 0.f;
    }
    w.A[a * npad + b] = v;
    w.B[a * npad + b] = (a == b) ? 1.f : 0.f;
  }
}

// The same for the identity permutation with n, ldh multiples of 4 and H
// 16-byte aligned: four consecutive outputs of a row are one aligned float4
// of the reversed source row, read backwards.
__global__ void __launch_bounds__(256) chol_gather_id4(const float* H, int64_t n, int64_t ldh,
                                                       int64_t npad, CholWs w) {
  const int64_t a = blockIdx.y;
  const float damp = (float)*w.damp;
  for (int64_t b = 4 * ((int64_t)blockIdx.x * 256 + threadIdx.x); b < npad; b += 4 * (int64_t)gridDim.x * 256) {
    float v[4], e[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) e[k] = (a == b + k) ? 1.f : 0.f;
    if (a < n && b < n) {
      const float4 x = *reinterpret_cast<const float4*>(H + (n - 1 - a) * ldh + (n - 4 - b));
      v[0] = x.w;
      v[1] = x.z;
      v[2] = x.y;
      v[3] = x.x;
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = (a == b + k) ? v[k] + damp : v[k];
      if (nonfinite_bits(v[0]) | nonfinite_bits(v[1]) | nonfinite_bits(v[2]) | nonfinite_bits(v[3]))
        mark_nonfinite(w);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = e[k];
    }
    *reinterpret_cast<float4*>(w.A + a * npad + b) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(w.B + a * npad + b) = make_float4(e[0], e[1], e[2], e[3]);
  }
}

// ------------------------------------------------------- diagonal block
//
// Factor the diagonal block S = A_pp = L L^T and invert L (fp64, one
// workgroup of four waves), blocked by SB = 32 columns.  With M_kk = L_kk^-1,
// X = L^-1 and the right-hand-side accumulators Bacc_ic = -sum_{k<i} L_ik X_kc:
//   for kb = 0..3:
//     B1 (wave 0): S_kk = L_kk L_kk^T and M_kk, two columns per step in
//        registers (lanes 0..31 hold the rows of S_kk, lanes 32..63 the
//        columns of the identity that becomes M_kk); the two current columns
//        of S_kk reach every lane through LDS.  No barrier inside.
//     P1: L_ik = S_ik M_kk^T (i > kb)   and   X_kb,c = M_kk Bacc_kb,c (c < kb)
//     P2: S_ij -= L_ik L_jk^T (kb < j <= i)   and
//         Bacc_ic -= L_ik X_kb,c (i > kb, c <= kb; X_kb,kb = M_kk)
// At the end row block i of L^-1 is X_i0 .. X_i,i-1, M_ii.  Only the lower
// triangle of S is read.  P1 and P2 are split into 16 x 16 output tiles
// (K = 32 on v_mfma_f64_16x16x4f64) dealt round-robin to the four waves.

constexpr int SB = 32;
constexpr int NSB = NB / SB;       // sub-blocks per side
constexpr int LDB = SB + 1;        // LDS row stride of a stored sub-block (doubles)
constexpr int BLKD = SB * LDB;     // doubles per stored sub-block

typedef double f64x4_t __attribute__((__vector_size__(4 * sizeof(double))));
typedef double f64x2_t __attribute__((ext_vector_type(2)));

// lower sub-block (i >= j) -> slot; strictly lower (i > c) -> accumulator slot
__device__ __forceinline__ int lslot(int i, int j) { return i * (i + 1) / 2 + j; }
__device__ __forceinline__ int bslot(int i, int c) { return i * (i - 1) / 2 + c; }

// Tile (ti, tj) of acc + sign * A B over K = 32, A(r, t) = pa[r * sar + t * sat],
// B(t, c) = pb[t * sbt + c * sbc] (LDS).  Lane l supplies A(16 ti + l % 16,
// k0 + l / 16) and B(k0 + l / 16, 16 tj + l % 16); register v holds element
// (16 ti + 4 v + l / 16, 16 tj + l % 16).
__device__ __forceinline__ f64x4_t tile_mma(f64x4_t acc, const double* pa, int sar, int sat,
                                            const double* pb, int sbt, int sbc, double sign, int ti,
                                            int tj) {
  const int l = threadIdx.x & 63, r = l & 15, kk = l >> 4;
#pragma unroll
  for (int k0 = 0; k0 < SB; k0 += 4) {
    const double av = sign * pa[(16 * ti + r) * sar + (k0 + kk) * sat];
    const double bv = pb[(k0 + kk) * sbt + (16 * tj + r) * sbc];
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc, 0, 0, 0);
  }
  return acc;
}

__device__ __forceinline__ f64x4_t tile_load(const double* blk, int ti, int tj) {
  const int l = threadIdx.x & 63;
  f64x4_t t;
#pragma unroll
  for (int v = 0; v < 4; ++v) t[v] = blk[(16 * ti + 4 * v + (l >> 4)) * LDB + 16 * tj + (l & 15)];
  return t;
}

__device__ __forceinline__ void tile_store(const f64x4_t& t, double* blk, int ti, int tj) {
  const int l = threadIdx.x & 63;
#pragma unroll
  for (int v = 0; v < 4; ++v) blk[(16 * ti + 4 * v + (l >> 4)) * LDB + 16 * tj + (l & 15)] = t[v];
}

// 1 / sqrt(x): hardware estimate refined by two Newton-Raphson steps
// y <- y (3 - x y^2) / 2 (each step doubles the correct bits)
__device__ __forceinline__ double rsqrt_nr(double x) {
  double y = __builtin_amdgcn_rsq(x);
  y = y * fma(-0.5 * x, y * y, 1.5);
  y = y * fma(-0.5 * x, y * y, 1.5);
  return y;
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
// B1 on one wave: factor the stored block Sk (lower triangle read) and
// overwrite it with M = L^-1 (lower triangular, zeros above).  Columns j and
// j + 1 are eliminated together: with d0 = S_jj, a = S_j+1,j, e = S_j+1,j+1 d0
// - a^2 (= d0 times the second pivot), y0 = 1/sqrt(d0), y1 = d0 y0 / sqrt(e),
// g = a / d0, every lane applies v[k] -= alpha c0[k] + beta c1[k] (k > j + 1)
// with beta = (v[j+1] - g v[j]) y1^2 and alpha = v[j] y0^2 - g beta, which is
// the rank-2 Cholesky update on the S rows and the forward substitution on the
// M columns; the M half then sets v[j] = v[j] y0, v[j+1] = (v[j+1] - g v[j]) y1.
// Lane r of the S half loads all of row r; its entries right of the diagonal
// (finite values of the stored block) only ever update other such entries of
// the same lane, so they never reach the factor.  Returns the first column
// whose pivot is not positive (or NaN), else -1; past a failed pivot the
// sweep continues with harmless values and its results are discarded.
// The two columns of a step reach every lane through LDS: col2 holds two
// buffers of 2 x SB doubles, step j's columns in buffer (j / 2) % 2, so that
// the S lanes can publish the next step's columns while this step's are still
// being read, and behind them two buffers that only the M lanes write to (no
// lane reads them), so that the publishing store needs no branch.  Each lane
// reads a column entry just before its update, kPre entries ahead, so the
// routine holds no copy of the columns.  All LDS accesses go through LDS-typed
// pointers off one base register (the buffers lie past the 64 KiB an
// immediate offset reaches from address zero; addressed one by one they cost
// a register move per read).  The routine stays out of line: inlined into the
// kernel, the register allocation spills.
constexpr int kPre = 8;

typedef __attribute__((address_space(3))) double lds_f64;
typedef __attribute__((address_space(3))) f64x2_t lds_f64x2;

__device__ __noinline__ int diag_factor32(double* Sk_, double* col2_) {
  const int l = threadIdx.x & 63, r = l & 31;
  const bool isS = l < 32;
  lds_f64* Sk = (lds_f64*)Sk_;
  // one base register for every column access (the buffers sit past the
  // 64 KiB reach of a read's immediate offset from address zero)
  unsigned cb = (unsigned)(size_t)(lds_f64*)col2_;
  asm volatile("" : "+v"(cb));
  lds_f64* col2 = (lds_f64*)(size_t)cb;
  // the M half publishes into two further, unread buffers (col2 + 4 SB ..
  // col2 + 8 SB), so the stores need no branch
  lds_f64* pub = col2 + (isS ? 0 : 4 * SB) + 2 * r;
  double v[SB];
#pragma unroll
  for (int k = 0; k < SB; ++k) v[k] = Sk[r * LDB + k];
#pragma unroll
  for (int k = 0; k < SB; ++k) v[k] = isS ? v[k] : (k == r ? 1.0 : 0.0);
  *(lds_f64x2*)pub = f64x2_t{v[0], v[1]};
  wave_sync_lds();
  // this step's pivot entries (S_jj, S_j+1,j; S_j+1,j+1)
  f64x2_t pv0 = *(const lds_f64x2*)(col2);
  f64x2_t pv1 = *(const lds_f64x2*)(col2 + 2);
  int bad = -1;
#pragma unroll
  for (int j = 0; j < SB; j += 2) {
    const lds_f64* cur = col2 + ((j / 2) & 1) * 2 * SB;
    const int nxo = (((j / 2) + 1) & 1) * 2 * SB;
    double d0 = pv0[0];
    const double a = pv1[0];
    if (!(d0 > 0.0)) {
      if (bad < 0) bad = j;
      d0 = 1.0;
    }
    double e = fma(pv1[1], d0, -a * a);
    if (!(e > 0.0)) {
      if (bad < 0) bad = j + 1;
      e = d0;
    }
    f64x2_t cn[2] = {f64x2_t{0.0, 0.0}, f64x2_t{0.0, 0.0}};
    if (j + 2 < SB) {
      cn[0] = *(const lds_f64x2*)(cur + 2 * (j + 2));
      cn[1] = *(const lds_f64x2*)(cur + 2 * (j + 3));
    }
    const double y0 = rsqrt_nr(d0), ye = rsqrt_nr(e);
    const double y0s = y0 * y0;
    const double g = a * y0s;
    const double y1 = ye * (d0 * y0);
    const double beta = fma(-g, v[j], v[j + 1]) * (y1 * y1);
    const double alpha = fma(v[j], y0s, -g * beta);
    if (j + 2 < SB) {
      v[j + 2] = fma(-alpha, cn[0][0], fma(-beta, cn[0][1], v[j + 2]));
      v[j + 3] = fma(-alpha, cn[1][0], fma(-beta, cn[1][1], v[j + 3]));
      *(lds_f64x2*)(pub + nxo) = f64x2_t{v[j + 2], v[j + 3]};
      wave_sync_lds();
      pv0 = *(const lds_f64x2*)(col2 + nxo + 2 * (j + 2));
      pv1 = *(const lds_f64x2*)(col2 + nxo + 2 * (j + 3));
    }
    f64x2_t cbuf[kPre];
#pragma unroll
    for (int k = j + 4; k < SB && k < j + 4 + kPre; ++k)
      cbuf[(k - j - 4) % kPre] = *(const lds_f64x2*)(cur + 2 * k);
#pragma unroll
    for (int k = j + 4; k < SB; ++k) {
      const f64x2_t t = cbuf[(k - j - 4) % kPre];
      if (k + kPre < SB) cbuf[(k - j - 4) % kPre] = *(const lds_f64x2*)(cur + 2 * (k + kPre));
      v[k] = fma(-alpha, t[0], fma(-beta, t[1], v[k]));
    }
    // the M half's columns j, j + 1 (the S half never reads them again)
    const double xj = v[j] * y0;
    v[j + 1] = fma(-g, v[j], v[j + 1]) * y1;
    v[j] = xj;
  }
  if (!isS) {
#pragma unroll
    for (int i = 0; i < SB; ++i) Sk[i * LDB + r] = v[i];
  }
  return bad;
}

// Step kb's trailing update except the diagonal block kb + 1: S_ij -= L_ik
// L_jk^T (kb < j <= i, (i, j) != (kb + 1, kb + 1)) and Bacc_ic -= L_ik X_kb,c
// (i > kb, c <= kb; X_kb,kb = M_kk), as 16 x 16 tiles dealt round-robin to
// `nw` waves (this one is number `w0`).
__device__ __forceinline__ void p2_rest(int kb, int w0, int nw, double* Ls, double* Bs) {
  const double* Mk = Ls + lslot(kb, kb) * BLKD;
  const int q = NSB - 1 - kb;
  const int nS = q * (q + 1) / 2, nB = q * (kb + 1);
  for (int job = w0; job < 4 * (nS + nB); job += nw) {
    const int prod = job >> 2, ti = (job >> 1) & 1, tj = job & 1;
    if (prod < nS) {
      int a = 0, u = prod;
      while (u > a) { u -= a + 1; ++a; }
      const int i = kb + 1 + a, j = kb + 1 + u;   // S_ij -= L_ik L_jk^T
      if (i == kb + 1 && j == kb + 1) continue;   // done before B1 of step kb + 1
      double* Sij = Ls + lslot(i, j) * BLKD;
      f64x4_t acc = tile_load(Sij, ti, tj);
      acc = tile_mma(acc, Ls + lslot(i, kb) * BLKD, LDB, 1, Ls + lslot(j, kb) * BLKD, 1, LDB, -1.0,
                     ti, tj);
      tile_store(acc, Sij, ti, tj);
    } else {
      const int pb = prod - nS;
      const int i = kb + 1 + pb / (kb + 1), c = pb % (kb + 1);   // Bacc_ic -= L_ik X_kb,c
      double* Bic = Bs + bslot(i, c) * BLKD;
      f64x4_t acc = (c == kb) ? f64x4_t{0.0, 0.0, 0.0, 0.0} : tile_load(Bic, ti, tj);
      const double* X = (c == kb) ? Mk : Ls + lslot(kb, c) * BLKD;
      acc = tile_mma(acc, Ls + lslot(i, kb) * BLKD, LDB, 1, X, LDB, 1, -1.0, ti, tj);
      tile_store(acc, Bic, ti, tj);
    }
  }
}

// LDS of the diagonal step
constexpr int kLsD = NSB * (NSB + 1) / 2 * BLKD;   // S, then L (below) / M (diagonal) / X
constexpr int kBsD = NSB * (NSB - 1) / 2 * BLKD;   // Bacc_ic, i > c

__device__ __forceinline__ void diag_step(int64_t npad, int64_t n, int p, const CholWs& w, double* Ls,
                                          double* Bs, double* col2, int& s_bad) {
  const int tid = threadIdx.x, wave = tid >> 6;

  // ---- load the lower sub-blocks of A_pp (fp32 -> fp64)
  {
    const float* Ap = w.A + (int64_t)p * NB * npad + (int64_t)p * NB;
    constexpr int PER = SB * SB / 4;                         // float4 per sub-block
    for (int e = tid; e < NSB * (NSB + 1) / 2 * PER; e += 256) {
      const int blk = e / PER, rem = e % PER;
      const int r = rem / (SB / 4), c4 = (rem % (SB / 4)) * 4;
      const int bi = blk >= 6 ? 3 : blk >= 3 ? 2 : blk >= 1 ? 1 : 0;
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

  for (int kb = 0; kb < NSB; ++kb) {
    // ---- B1 on wave 0; meanwhile waves 1..3 finish the trailing update of
    // step kb - 1 (all but the diagonal block kb, which B1 reads)
    if (wave == 0) {
      const int bad = diag_factor32(Ls + lslot(kb, kb) * BLKD, col2);
      if (tid == 0 && bad >= 0) s_bad = SB * kb + bad;
    } else if (kb > 0) {
      p2_rest(kb - 1, wave - 1, 3, Ls, Bs);
    }
    __syncthreads();
    if (s_bad >= 0) break;
    const double* Mk = Ls + lslot(kb, kb) * BLKD;
    // ---- P1: 3 products x 4 tiles; results held until every wave has read
    // the blocks they overwrite
    {
      f64x4_t res[3];
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        const int job = wave + 4 * u, prod = job >> 2, ti = (job >> 1) & 1, tj = job & 1;
        f64x4_t acc = f64x4_t{0.0, 0.0, 0.0, 0.0};
        if (prod < NSB - 1 - kb) {
          const int i = kb + 1 + prod;   // L_ik = S_ik M_kk^T
          acc = tile_mma(acc, Ls + lslot(i, kb) * BLKD, LDB, 1, Mk, 1, LDB, 1.0, ti, tj);
        } else {
          const int c = prod - (NSB - 1 - kb);   // X_kb,c = M_kk Bacc_kb,c
          acc = tile_mma(acc, Mk, LDB, 1, Bs + bslot(kb, c) * BLKD, LDB, 1, 1.0, ti, tj);
        }
        res[u] = acc;
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        const int job = wave + 4 * u, prod = job >> 2, ti = (job >> 1) & 1, tj = job & 1;
        double* out = (prod < NSB - 1 - kb) ? Ls + lslot(kb + 1 + prod, kb) * BLKD
                                            : Ls + lslot(kb, prod - (NSB - 1 - kb)) * BLKD;
        tile_store(res[u], out, ti, tj);
      }
    }
    __syncthreads();
    // ---- the next diagonal block's share of the trailing update, S_k+1,k+1
    // -= L_k+1,k L_k+1,k^T (one tile per wave), so that B1 can start on it
    if (kb + 1 < NSB) {
      const int ti = wave >> 1, tj = wave & 1, i = kb + 1;
      double* Sii = Ls + lslot(i, i) * BLKD;
      f64x4_t acc = tile_load(Sii, ti, tj);
      acc = tile_mma(acc, Ls + lslot(i, kb) * BLKD, LDB, 1, Ls + lslot(i, kb) * BLKD, 1, LDB, -1.0, ti, tj);
      tile_store(acc, Sii, ti, tj);
      __syncthreads();
    }
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

  // ---- Linv (fp32, NB x NB, zeros above the diagonal), 4 columns per store
  for (int e = tid; e < NB * NB / 4; e += 256) {
    const int r = e / (NB / 4), c = (e % (NB / 4)) * 4;
    const int bi = r / SB, bj = c / SB, rr = r % SB, cc = c % SB;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (bi >= bj) {
      const double* src = Ls + lslot(bi, bj) * BLKD + rr * LDB + cc;
      v = make_float4((float)src[0], (float)src[1], (float)src[2], (float)src[3]);
    }
    *reinterpret_cast<float4*>(linv_buf(w, p & 1) + (int64_t)r * NB + c) = v;
  }
}

// ------------------------------------------------------- tile products

// Layout of a global operand tile: element (x, k) of an X x K operand.
//   XK: stored row-major as [x][k] (leading dimension ld)
//   KX: stored row-major as [k][x]
enum { XK = 0, KX = 1 };

// A stage is KS values of k for X consecutive x, held in LDS as sT[k][x]
// (stride ST = X + 1, odd: conflict-free transposed stores).  gload fetches a
// thread's share of it (16-byte loads) into registers; lstore writes those
// registers to LDS.
template <int X>
constexpr int stage_vecs() { return (X * KS / 4) / 256; }

template <int LAY, int X>
__device__ inline void gload(float4 (&r)[stage_vecs<X>()], const float* G, int64_t ld, int k0) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < stage_vecs<X>(); ++q) {
    const int idx = tid + 256 * q;
    if (LAY == XK) {
      const int x = idx >> 3, k4 = (idx & 7) * 4;
      r[q] = *reinterpret_cast<const float4*>(G + (int64_t)x * ld + k0 + k4);
    } else {
      const int k = idx / (X / 4), x4 = (idx % (X / 4)) * 4;
      r[q] = *reinterpret_cast<const float4*>(G + (int64_t)(k0 + k) * ld + x4);
    }
  }
}

template <int LAY, int X, int ST = X + 1>
__device__ inline void lstore(float* sT, const float4 (&r)[stage_vecs<X>()]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < stage_vecs<X>(); ++q) {
    const int idx = tid + 256 * q;
    if (LAY == XK) {
      const int x = idx >> 3, k4 = (idx & 7) * 4;
      sT[(k4 + 0) * ST + x] = r[q].x;
      sT[(k4 + 1) * ST + x] = r[q].y;
      sT[(k4 + 2) * ST + x] = r[q].z;
      sT[(k4 + 3) * ST + x] = r[q].w;
    } else {
      const int k = idx / (X / 4), x4 = (idx % (X / 4)) * 4;
      sT[k * ST + x4 + 0] = r[q].x;
      sT[k * ST + x4 + 1] = r[q].y;
      sT[k * ST + x4 + 2] = r[q].z;
      sT[k * ST + x4 + 3] = r[q].w;
    }
  }
}

// LDS of a tile product with MR x MC output: all of K for both operands
constexpr size_t tile_lds(int MR, int MC) { return (size_t)NB * (MR + 1 + MC + 1) * sizeof(float); }
constexpr size_t kTileLdsFull = tile_lds(128, 128);   // U2 tiles
constexpr size_t kTileLdsQuarter = tile_lds(128, 32);  // PL, PY, U1 quarter tiles

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

  // All of K at once: every thread issues its loads of all NB / KS stages
  // before the first is written to LDS, so the global latency is paid once;
  // one barrier, then the MFMAs run with no further waits on memory.
  template <int LA, int LB>
  __device__ void run(const float* Ag, int64_t lda, const float* Bg, int64_t ldb, float* sm) {
    constexpr int NS = NB / KS, SA = MR + 1, SBT = MC + 1;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / WC, wn = wave % WC;
    const int lr = lane & 31, lk = lane >> 5;
    float* sA = sm;              // NB x SA: sA[k][x]
    float* sB = sm + NB * SA;    // NB x SBT
    {
      float4 ra[NS][stage_vecs<MR>()], rb[NS][stage_vecs<MC>()];
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        gload<LA, MR>(ra[st], Ag, lda, st * KS);
        gload<LB, MC>(rb[st], Bg, ldb, st * KS);
      }
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        lstore<LA, MR, SA>(sA + st * KS * SA, ra[st]);
        lstore<LB, MC, SBT>(sB + st * KS * SBT, rb[st]);
      }
    }
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < NB; kk += 2) {
      float af[TR], bf[TC];
#pragma unroll
      for (int a = 0; a < TR; ++a) af[a] = sA[(kk + lk) * SA + (wm * TR + a) * 32 + lr];
#pragma unroll
      for (int b = 0; b < TC; ++b) bf[b] = sB[(kk + lk) * SBT + (wn * TC + b) * 32 + lr];
#pragma unroll
      for (int a = 0; a < TR; ++a)
#pragma unroll
        for (int b = 0; b < TC; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[a], bf[b], acc[a][b], 0, 0, 0);
    }
  }

  // MODE 0: C = acc; MODE 1: C -= acc.  32x32 accumulator layout: lane holds
  // column lane % 32; register v holds row 8 * (v / 4) + 4 * (lane / 32) + v % 4.
  // In MODE 1 every old value is loaded before the first store (written as
  // one load per element followed by its store, the compiler would keep them
  // in order, one memory round trip per element, as it cannot rule out that
  // two elements alias).
  template <int MODE>
  __device__ void store(float* C, int64_t ldc) const {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / WC, wn = wave % WC;
    const int lr = lane & 31, lk = lane >> 5;
    float old[TR][TC][16];
    if (MODE == 1) {
#pragma unroll
      for (int a = 0; a < TR; ++a)
#pragma unroll
        for (int b = 0; b < TC; ++b)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int r = (wm * TR + a) * 32 + 8 * (v >> 2) + 4 * lk + (v & 3);
            const int c = (wn * TC + b) * 32 + lr;
            old[a][b][v] = C[(int64_t)r * ldc + c];
          }
    }
#pragma unroll
    for (int a = 0; a < TR; ++a)
#pragma unroll
      for (int b = 0; b < TC; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = (wm * TR + a) * 32 + 8 * (v >> 2) + 4 * lk + (v & 3);
          const int c = (wn * TC + b) * 32 + lr;
          C[(int64_t)r * ldc + c] = MODE == 0 ? acc[a][b][v] : old[a][b][v] - acc[a][b][v];
        }
  }
};

// Step p's panels, as quarter tiles (128 x 32): PL, Lp_i = A_ip Linv^T for i
// > p (the first 4 (P - p - 1) workgroups), and PY, Yp_c = Linv B_pc for c <=
// p (the next 4 (p + 1)).  Buffers of parity p % 2.
__global__ void __launch_bounds__(256) chol_panel(int64_t npad, int P, int p, CholWs w) {
  if (*w.flag) return;
  extern __shared__ __align__(16) float sm[];
  const int npl = 4 * (P - p - 1);
  const bool pl = (int)blockIdx.x < npl;
  const int u = pl ? blockIdx.x : blockIdx.x - npl;
  const int t = u >> 2, quarter = u & 3;
  const float* Linv = linv_buf(w, p & 1);
  TileMma<4, 1, 1, 1> mm;
  mm.zero();
  if (pl) {
    const int i = p + 1 + t;
    const float* Aip = w.A + (int64_t)i * NB * npad + (int64_t)p * NB;
    // B(j, k) = Linv[32 quarter + j][k]
    mm.run<XK, XK>(Aip, npad, Linv + (int64_t)32 * quarter * NB, NB, sm);
    mm.store<0>(lp_buf(w, p % NBO) + (int64_t)i * NB * NB + 32 * quarter, NB);
  } else {
    const int c = t;
    // A(i, k) = Linv[i][k]; B(j, k) = B[p NB + k][c NB + 32 quarter + j]
    const float* Bpc = w.B + (int64_t)p * NB * npad + (int64_t)c * NB + 32 * quarter;
    mm.run<XK, KX>(Linv, NB, Bpc, npad, sm);
    mm.store<0>(yp_buf(w, p % NBO) + (int64_t)c * NB + 32 * quarter, npad);
  }
}

// U2 of step p with the step's panel p's outer block ending at panel `bend`
// (the last panel, P - 1, when the sweep is one-level): the SYRK tiles
// A_ij -= Lp_i Lp_j^T for p + 2 <= j <= bend, i >= j, then the forward-
// substitution tiles B_ic -= Lp_i Yp_c for p < i <= bend, c <= p, then the copy
// of Y_p into row block p of B.  The columns and rows past `bend` get panel p's
// share from the outer update of its block.
__host__ __device__ inline int u2_syrk_tiles(int P, int p, int bend) {
  int cnt = 0;
  for (int j = p + 2; j <= bend; ++j) cnt += P - j;
  return cnt;
}

__host__ __device__ inline int u2_tiles(int P, int p, int bend) {
  return u2_syrk_tiles(P, p, bend) + (bend - p) * (p + 1) + (p + 1);
}

// `sm` holds kTileLdsFull bytes.
__device__ __forceinline__ void u2_tile(int64_t npad, int P, int p, int bend, int t, const CholWs& w,
                                        float* sm) {
  const float* Lp = lp_buf(w, p % NBO);
  const float* Yp = yp_buf(w, p % NBO);
  const int nsyrk = u2_syrk_tiles(P, p, bend);
  const int nfwd = (bend - p) * (p + 1);
  if (t < nsyrk + nfwd) {
    TileMma<2, 2, 2, 2> mm;
    mm.zero();
    if (t < nsyrk) {
      int j = p + 2;
      while (t >= P - j) { t -= P - j; ++j; }
      const int i = j + t;   // j <= i
      mm.run<XK, XK>(Lp + (int64_t)i * NB * NB, NB, Lp + (int64_t)j * NB * NB, NB, sm);
      mm.store<1>(w.A + (int64_t)i * NB * npad + (int64_t)j * NB, npad);
    } else {
      t -= nsyrk;
      const int i = p + 1 + t / (p + 1), c = t % (p + 1);
      mm.run<XK, KX>(Lp + (int64_t)i * NB * NB, NB, Yp + (int64_t)c * NB, npad, sm);
      mm.store<1>(w.B + (int64_t)i * NB * npad + (int64_t)c * NB, npad);
    }
  } else {
    const int c = t - nsyrk - nfwd;   // copy tile c of Y_p
    const float* src = Yp + (int64_t)c * NB;
    float* dst = w.B + (int64_t)p * NB * npad + (int64_t)c * NB;
    for (int e = threadIdx.x; e < NB * NB / 4; e += 256) {
      const int r = e / (NB / 4), c4 = (e % (NB / 4)) * 4;
      *reinterpret_cast<float4*>(dst + (int64_t)r * npad + c4) =
          *reinterpret_cast<const float4*>(src + (int64_t)r * npad + c4);
    }
  }
}

// Step p of the sweep, one launch: workgroup 0 factors and inverts diagonal
// block p (if p < P); the others run U2 of step p - 1, which writes only
// columns past p and row blocks past p - 1 of B, so it overlaps the diagonal
// block.  The U2 tiles reuse the diagonal step's LDS for their stages.
__global__ void __launch_bounds__(256) chol_step(int64_t npad, int64_t n, int P, int p, int bend_prev,
                                                 CholWs w) {
  if (*w.flag) return;
  __shared__ __align__(16) double lds[kLsD + kBsD + 8 * SB];
  __shared__ int s_bad;
  static_assert(sizeof(lds) >= kTileLdsFull, "a U2 tile fits the diagonal step's LDS");
  if (blockIdx.x > 0) {
    u2_tile(npad, P, p - 1, bend_prev, (int)blockIdx.x - 1, w, reinterpret_cast<float*>(lds));
    return;
  }
  if (p < P) diag_step(npad, n, p, w, lds, lds + kLsD, lds + kLsD + kBsD, s_bad);
}

// U1 of step p: the SYRK tiles of column p + 1, A_i,p+1 -= Lp_i Lp_p+1^T for
// i > p, as 128 x 32 quarter tiles (four times the workgroups, a quarter of
// the latency, for the kernel on the critical path).
__global__ void __launch_bounds__(256) chol_u1(int64_t npad, int p, CholWs w) {
  if (*w.flag) return;
  extern __shared__ __align__(16) float sm[];
  const float* Lp = lp_buf(w, p % NBO);
  const int t = blockIdx.x;
  TileMma<4, 1, 1, 1> mm;
  mm.zero();
  const int quarter = t & 3;
  const int i = p + 1 + (t >> 2), j = p + 1;
  mm.run<XK, XK>(Lp + (int64_t)i * NB * NB, NB, Lp + (int64_t)j * NB * NB + 32 * quarter * NB, NB, sm);
  mm.store<1>(w.A + (int64_t)i * NB * npad + (int64_t)j * NB + 32 * quarter, npad);
}

// Outer update of the outer block of panels b0 .. b0 + NBO - 1 (two-level
// sweep), once its last panel's L and Y are out: every column and row block
// past the block gets the block's share at once, with K = NBO * NB:
//   SYRK  A_ij -= sum_q L_i,b0+q L_j,b0+q^T            (j >= b1 = b0 + NBO, i >= j)
//   fwd   B_ic -= sum_{q: b0+q >= c} L_i,b0+q Y_b0+q,c  (i >= b1, c < b1)
// A right-looking sweep reads and writes the whole trailing matrix once per
// panel; with rank-512 updates it does so once per outer block, and each
// tile's read-modify-write is amortized over four times the products.
//
// The products run on the bf16 matrix cores at fp32 accuracy: every fp32
// operand is split exactly into three bf16 parts, x = x1 + x2 + x3 (8 + 8 + 8
// significant bits), and a b = sum of the six products a_i b_j with i + j <= 4
// (the three dropped ones are below 2^-24 |a b|).  bf16 products are exact in
// fp32; a1 b1 accumulates in one fp32 accumulator and the five smaller terms
// in another, so the accumulation rounds as often as an fp32 product would.
// Six v_mfma_f32_32x32x16_bf16 (32 cycles each) replace eight
// v_mfma_f32_32x32x2f32 (64 cycles each) per 32 x 32 x 16 step.
//
// The split is made once per outer block (chol_presplit: every panel feeds
// all the tiles of its row or column block, which split it again each when
// the tiles split their own operands).  One 128 x 128 output tile per
// workgroup (four waves as 2 x 2, each 64 x 64 as 2 x 2 accumulator pairs),
// two workgroups per CU.  K runs in stages of 16 through a ring of three LDS
// stages filled by direct-to-LDS loads, two stages in flight while one is
// multiplied; a stage holds the three parts of both operands k-major with the
// rows' 16-byte chunks swizzled by k, read transposed into the MFMA layout.
// (Staged 32 at a time through registers, with two barriers and a store
// phase per stage, the n = 28672 factor took 111 ms; this way 101 ms.  A
// ring of three 32-k stages needs 144 KiB, one workgroup per CU: 115 ms.)

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// two fp32 values -> two bf16 rounded to nearest (one v_cvt_pk_bf16_f32),
// packed low then high
__device__ __forceinline__ uint32_t pack_bf16(f32x2_t v) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
// the two bf16 of a packed word, widened (exactly) to fp32
__device__ __forceinline__ f32x2_t unpack_bf16(uint32_t u) {
  return f32x2_t{__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u)};
}

// a pair x = x1 + x2 + x3 exactly, each part packed for the pair (each
// remainder is exact in fp32): 11 VALU operations for two values, where the
// rounding done in integer arithmetic took about 40
__device__ __forceinline__ void split3_pair(f32x2_t x, uint32_t& h, uint32_t& m, uint32_t& l) {
  h = pack_bf16(x);
  const f32x2_t r1 = x - unpack_bf16(h);
  m = pack_bf16(r1);
  const f32x2_t r2 = r1 - unpack_bf16(m);
  l = pack_bf16(r2);
}

// The bf16 parts of an outer block's panels, made once for all of its outer
// update's tiles (each panel feeds every tile of its row or column block),
// k-major like Y: [slot][k / 32][part][k % 32][row or column], so that a
// tile's stage holds, per part and k, 256 contiguous bytes of its 128 rows.
// L slot q rows r0 .. npad - 1 (transposed through LDS, 32 rows a
// workgroup: workgroups [0, nL)); Y slot q columns 0 .. c1 - 1 (already
// k-major: 1024 columns of one k a workgroup).
__device__ __forceinline__ int64_t kmaj_at(int64_t npad, int q, int part, int k, int64_t row) {
  return ((int64_t)((q * (NB / 32) + k / 32) * 3 + part) * 32 + (k % 32)) * npad + row;
}

__global__ void __launch_bounds__(256) chol_presplit(int64_t npad, int64_t r0, int64_t c1, int nL,
                                                     CholWs w) {
  if (*w.flag) return;
  __shared__ float tile[32][NB + 1];
  const int tid = threadIdx.x;
  if ((int)blockIdx.x < nL) {
    const int64_t ntiles = (npad - r0) / 32;   // npad - r0 is a multiple of NB
    const int q = (int)(blockIdx.x / ntiles);
    const int64_t row0 = r0 + (blockIdx.x % ntiles) * 32;
    const float* src = lp_buf(w, q) + row0 * NB;
    // 32 rows x 128 k: float4 u of a thread is row tid / 8, k (tid % 8) * 16 + 4 u
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = tid >> 3, k = (tid & 7) * 16 + 4 * u;
      const float4 x = *reinterpret_cast<const float4*>(src + r * NB + k);
      tile[r][k] = x.x;
      tile[r][k + 1] = x.y;
      tile[r][k + 2] = x.z;
      tile[r][k + 3] = x.w;
    }
    __syncthreads();
    // k = tid % 128, rows (tid / 128) * 16 .. + 15: eight pairs of rows
    const int k = tid & (NB - 1), rb = (tid >> 7) * 16;
    uint32_t h[8], m[8], l[8];
#pragma unroll
    for (int v = 0; v < 8; ++v)
      split3_pair(f32x2_t{tile[rb + 2 * v][k], tile[rb + 2 * v + 1][k]}, h[v], m[v], l[v]);
    const uint32_t* pp[3] = {h, m, l};
#pragma unroll
    for (int part = 0; part < 3; ++part) {
      unsigned short* dst = w.Ls + kmaj_at(npad, q, part, k, row0 + rb);
      *reinterpret_cast<uint4*>(dst) = make_uint4(pp[part][0], pp[part][1], pp[part][2], pp[part][3]);
      *reinterpret_cast<uint4*>(dst + 8) = make_uint4(pp[part][4], pp[part][5], pp[part][6], pp[part][7]);
    }
    return;
  }
  // Y: 1024 consecutive columns of one k of slot q, four a thread
  const int64_t b = blockIdx.x - nL;
  const int64_t nch = (c1 + 1023) / 1024;
  const int q = (int)(b / (NB * nch));
  const int k = (int)((b / nch) % NB);
  const int64_t col = (b % nch) * 1024 + 4 * tid;
  if (col >= c1) return;
  const float4 x = *reinterpret_cast<const float4*>(yp_buf(w, q) + (int64_t)k * npad + col);
  uint32_t h0, m0, l0, h1, m1, l1;
  split3_pair(f32x2_t{x.x, x.y}, h0, m0, l0);
  split3_pair(f32x2_t{x.z, x.w}, h1, m1, l1);
  *reinterpret_cast<uint2*>(w.Ys + kmaj_at(npad, q, 0, k, col)) = make_uint2(h0, h1);
  *reinterpret_cast<uint2*>(w.Ys + kmaj_at(npad, q, 1, k, col)) = make_uint2(m0, m1);
  *reinterpret_cast<uint2*>(w.Ys + kmaj_at(npad, q, 2, k, col)) = make_uint2(l0, l1);
}

// chunk swizzle {0, 6, 12, 10}[k % 4] of the 16-byte chunks of an LDS k-row:
// the transposing operand reads of 16 lanes (4 values of k x 16 rows) then
// fall on distinct banks
__device__ __forceinline__ int ko_swz(int k) { return (0xAC60 >> (4 * (k & 3))) & 15; }

typedef short ko_i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) ko_i16x4_t ko_lds_i16x4_t;

// 4 values of k of one row, transposed out of the k-major stage
__device__ __forceinline__ ko_i16x4_t ko_ld(const unsigned short* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((ko_lds_i16x4_t*)p);
}

// Ring of three stages for the outer update, each a distinct LDS object (the
// A and B operands of 32 values of k, three bf16 parts each, 48 KiB), so that
// the compiler's tracking of direct-to-LDS loads sees that refilling one slot
// does not alias the reads of another.
constexpr int RKS = 16;   // k per ring stage
struct OuterSlot {
  unsigned short a[3 * RKS * NB];
  unsigned short b[3 * RKS * NB];
};
__shared__ __align__(16) OuterSlot co_s0, co_s1, co_s2;

template <int SLOT>
__device__ __forceinline__ OuterSlot& co_slot() {
  if constexpr (SLOT == 0) return co_s0;
  else if constexpr (SLOT == 1) return co_s1;
  else return co_s2;
}

typedef __attribute__((address_space(3))) void co_lds_void_t;

// s_waitcnt immediate: at most `vm` loads in flight (vmcnt, 6 bits split over
// [3:0] and [15:14]), expcnt unconstrained, at most `lgkm` LDS operations
constexpr int co_cnt(int vm, int lgkm) { return (vm & 15) | (7 << 4) | (lgkm << 8) | ((vm >> 4) << 14); }

// the empty asm hides the offset from the optimizer, so that the stage base
// is added at each load instead of one live address per slot and load
__device__ __forceinline__ uint32_t co_opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

struct OuterCtx {
  const unsigned char* ga;   // split parts of the A tile's rows, stage 0 (bytes)
  const unsigned char* gb;   // same for the B tile
  int64_t stage_bytes;       // bytes from one 32-k stage of the split panels to the next
  uint32_t off[3];           // byte offsets of the lane's three loads within a stage
  int wave;
  int rdA0, rdA1, rdB0, rdB1;
};

// Stage k0 into slot SLOT: wave w loads chunks h = 6 w .. 6 w + 5 of each
// operand (part h / 8, k rows 4 (h % 8) .. + 3, 1 KiB); lane l of a chunk
// lands at k row 4 (h % 8) + l / 16, 16-byte position l % 16, and fetches the
// rows that position holds under the swizzle, 8 ((l % 16) ^ swz(k)) .. + 7.
template <int SLOT>
__device__ __forceinline__ void co_issue(const OuterCtx& c, int kst) {
  OuterSlot& sl = co_slot<SLOT>();
  const int64_t sb = ((int64_t)(kst >> 1) * 96 + (kst & 1) * 16) * c.stage_bytes;
  const unsigned char* ga = c.ga + sb;
  const unsigned char* gb = c.gb + sb;
#pragma unroll
  for (int u = 0; u < 3; ++u) {
    const int h = 3 * c.wave + u;
    const int e = ((h >> 2) * RKS + 4 * (h & 3)) * NB;
    __builtin_amdgcn_global_load_lds((const void*)(ga + co_opaque(c.off[u])), (co_lds_void_t*)(sl.a + e), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((const void*)(gb + co_opaque(c.off[u])), (co_lds_void_t*)(sl.b + e), 16, 0, 0);
  }
}

// the 48 products of one stage (two steps of 16 k) from slot SLOT
template <int SLOT>
__device__ __forceinline__ void co_mma(const OuterCtx& c, f32x16_t (&hi)[2][2], f32x16_t (&lo)[2][2]) {
  const OuterSlot& sl = co_slot<SLOT>();
#pragma unroll
  for (int ks = 0; ks < RKS; ks += 16) {
    bf16x8_t af[2][3], bf[2][3];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int pt = 0; pt < 3; ++pt) {
        const unsigned short* q = sl.a + pt * RKS * NB + ks * NB + (a ? c.rdA1 : c.rdA0);
        af[a][pt] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(ko_ld(q), ko_ld(q + 4 * NB), 0, 1, 2,
                                                                         3, 4, 5, 6, 7));
      }
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int pt = 0; pt < 3; ++pt) {
        const unsigned short* q = sl.b + pt * RKS * NB + ks * NB + (b ? c.rdB1 : c.rdB0);
        bf[b][pt] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(ko_ld(q), ko_ld(q + 4 * NB), 0, 1, 2,
                                                                         3, 4, 5, 6, 7));
      }
    // term order: each group of four MFMAs updates four different accumulators
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
        hi[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a][0], bf[b][0], hi[a][b], 0, 0, 0);
#pragma unroll
    for (int term = 0; term < 5; ++term) {
      const int pa = term == 0 ? 0 : term == 1 ? 1 : term == 2 ? 0 : term == 3 ? 1 : 2;
      const int pb = term == 0 ? 1 : term == 1 ? 0 : term == 2 ? 2 : term == 3 ? 1 : 0;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          lo[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a][pa], bf[b][pb], lo[a][b], 0, 0, 0);
    }
  }
}

// Stage s of nst in slot K = s % 3: wait until this wave's loads of stage s
// have landed (stage s + 1's twelve may still be in flight) and its reads of
// stage s - 1 have returned, meet the other waves (every wave's loads of stage
// s have landed and every read of slot (s + 2) % 3 is done), refill that slot
// with stage s + 2, then multiply stage s.  No branch: past the end the refill
// loads the last stage again (in bounds, never read).
template <int K>
__device__ __forceinline__ void co_step(const OuterCtx& c, int s, int nst, f32x16_t (&hi)[2][2],
                                        f32x16_t (&lo)[2][2]) {
  __builtin_amdgcn_s_waitcnt(co_cnt(6, 0));
  __builtin_amdgcn_s_barrier();
  co_issue<(K + 2) % 3>(c, min(s + 2, nst - 1));
  co_mma<K>(c, hi, lo);
}

__global__ void __launch_bounds__(256, 2) chol_outer(int64_t npad, int P, int b0, CholWs w) {
  if (*w.flag) return;
  const int b1 = b0 + NBO;
  // Tiles in 8 x 8 super-tiles, one super-tile per XCD at a time: workgroup
  // b runs on XCD b % 8, so its slot b / 8 on that XCD takes tile b / 8 % 64
  // of super-tile 8 (b / 512) + b % 8.  The 64 workgroups an XCD holds then
  // share 8 row blocks and 8 column blocks of operands in its L2 (in launch
  // order they were 64 row blocks of one column block).  Super-tiles: the
  // SYRK triangle (i >= j >= b1) by super-rows, then the fwd rectangle
  // (i >= b1, c < b1); tiles outside them (past the edges, above the
  // diagonal, and the padding of the super-tile count to a multiple of 8)
  // exit at once.
  const int q2 = P - b1;
  const int T = (q2 + 7) / 8, Cs = (b1 + 7) / 8;
  const int nsS = T * (T + 1) / 2;
  const int slot = blockIdx.x / 8;
  const int st = 8 * (slot / 64) + blockIdx.x % 8;
  const int di = (slot % 64) / 8, dj = slot % 8;
  const bool fwd = st >= nsS;
  int i, j, qlo = 0;
  if (!fwd) {
    int si = 0;
    while ((si + 1) * (si + 2) / 2 <= st) ++si;
    const int sj = st - si * (si + 1) / 2;
    i = b1 + 8 * si + di;
    j = b1 + 8 * sj + dj;
    if (i >= P || j > i) return;
  } else {
    const int sp = st - nsS;
    if (sp >= T * Cs) return;
    i = b1 + 8 * (sp / Cs) + di;
    j = 8 * (sp % Cs) + dj;           // the column block c of B
    if (i >= P || j >= b1) return;
    qlo = j > b0 ? j - b0 : 0;        // panels b0 + q >= c
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lk = lane >> 5;
  f32x16_t hi[2][2], lo[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        hi[a][b][v] = 0.f;
        lo[a][b][v] = 0.f;
      }
  // A rows i NB .. + 127 of L_b0+q; B rows j NB .. + 127 of L_b0+q (SYRK) or
  // columns j NB .. + 127 of Y_b0+q (fwd); q = k / NB, panel q in slot q (b0
  // is a multiple of NBO).  Stage k0 of the split panels starts (k0 / 32) 96
  // npad elements in (kmaj_at).
  OuterCtx c;
  c.ga = reinterpret_cast<const unsigned char*>(w.Ls + (int64_t)i * NB);
  c.gb = reinterpret_cast<const unsigned char*>((fwd ? w.Ys : w.Ls) + (int64_t)j * NB);
  c.stage_bytes = npad * 2;   // bytes of one k row of the split panels
  c.wave = wave;
#pragma unroll
  for (int u = 0; u < 3; ++u) {
    const int h = 3 * wave + u;
    const int k = 4 * (h & 3) + (lane >> 4);
    const int row = ((lane & 15) ^ ko_swz(k)) << 3;
    c.off[u] = (uint32_t)((((int64_t)(h >> 2) * 32 + k) * npad + row) * 2);
  }
  // operand reads (the layout of v_mfma_f32_32x32x16_bf16: lane l takes row
  // l % 32 of the operand tile, k 8 (l / 32) .. + 7): within each 16 lanes,
  // lane jj addresses k kr = 8 (g / 2) + jj / 4 (+ 4 for the second read) and
  // rows fo = 16 (g % 2) + 4 (jj % 4) .. + 3 of the 32-row tile, g = lane / 16;
  // lane jj then receives 4 values of k of row 16 (g % 2) + jj.  The swizzle
  // of kr is that of kr + 4 and of kr + 16.
  const int rg = lane >> 4, rjj = lane & 15;
  const int kr = 8 * (rg >> 1) + (rjj >> 2);
  const int fo = 16 * (rg & 1) + 4 * (rjj & 3);
  auto rd_off = [&](int row) { return kr * NB + (((row >> 3) ^ ko_swz(kr)) << 3) + (row & 7); };
  c.rdA0 = rd_off(wm * 64 + fo);
  c.rdA1 = rd_off(wm * 64 + 32 + fo);
  c.rdB0 = rd_off(wn * 64 + fo);
  c.rdB1 = rd_off(wn * 64 + 32 + fo);
  const int ks0 = qlo * (NB / RKS);           // first stage
  const int nst = NBO * (NB / RKS) - ks0;     // 8, 16, 24 or 32 stages
  co_issue<0>(c, ks0);
  co_issue<1>(c, ks0 + 1);
  int s = 0;
  for (; s + 3 <= nst; s += 3) {
    co_step<0>(c, ks0 + s, ks0 + nst, hi, lo);
    co_step<1>(c, ks0 + s + 1, ks0 + nst, hi, lo);
    co_step<2>(c, ks0 + s + 2, ks0 + nst, hi, lo);
  }
  if (s < nst) co_step<0>(c, ks0 + s, ks0 + nst, hi, lo);
  if (s + 1 < nst) co_step<1>(c, ks0 + s + 1, ks0 + nst, hi, lo);
  // the refills past the end are still landing in LDS: drain them before the
  // workgroup can exit
  __builtin_amdgcn_s_waitcnt(co_cnt(0, 0));
  // C -= hi + lo, every old value of an accumulator tile loaded before its stores
  float* C = (fwd ? w.B : w.A) + (int64_t)i * NB * npad + (int64_t)j * NB;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      float old[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wm * 64 + 32 * a + 8 * (v >> 2) + 4 * lk + (v & 3);
        old[v] = C[(int64_t)r * npad + wn * 64 + 32 * b + lr];
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wm * 64 + 32 * a + 8 * (v >> 2) + 4 * lk + (v & 3);
        C[(int64_t)r * npad + wn * 64 + 32 * b + lr] = old[v] - (hi[a][b][v] + lo[a][b][v]);
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

// The same with n, ldr multiples of 4 and R 16-byte aligned: four outputs of a
// row from one aligned float4 of the reversed source row.
__global__ void __launch_bounds__(256) chol_flip4(int64_t n, int64_t npad, float* R, int64_t ldr,
                                                  CholWs w) {
  if (*w.flag) return;
  const int64_t a = blockIdx.y;
  for (int64_t b = 4 * ((int64_t)blockIdx.x * 256 + threadIdx.x); b < n; b += 4 * (int64_t)gridDim.x * 256) {
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (b + 3 >= a) {
      const float4 x = *reinterpret_cast<const float4*>(w.B + (n - 1 - a) * npad + (n - 4 - b));
      const float y[4] = {x.w, x.z, x.y, x.x};
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = (b + k >= a) ? y[k] : 0.f;
    }
    *reinterpret_cast<float4*>(R + a * ldr + b) = make_float4(v[0], v[1], v[2], v[3]);
  }
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
    if (!act_order && n % 4 == 0 && ldh % 4 == 0 && reinterpret_cast<uintptr_t>(H) % 16 == 0) {
      const unsigned gx = (unsigned)std::min<int64_t>((npad / 4 + 255) / 256, 64);
      hipLaunchKernelGGL(chol_gather_id4, dim3(gx, (unsigned)npad), dim3(256), 0, s, H, n, ldh, npad, w);
    } else {
      const unsigned gx = (unsigned)std::min<int64_t>((npad + 255) / 256, 64);
      hipLaunchKernelGGL(chol_gather, dim3(gx, (unsigned)npad), dim3(256), 0, s, H, n, ldh,
                         (const int32_t*)perm, npad, w);
    }
    KQ_LAUNCHED("chol_gather");
  }
  // one stream: step p (diagonal block p with U2 of step p - 1), the panels
  // of step p, then U1 of step p or, after the last panel of an outer block,
  // the block's outer update; a last step launch runs U2 of step P - 1.  The
  // sweep is two-level (outer blocks of NBO panels) from kTwoLevelMinPanels
  // panels on; below that every U2 covers the whole trailing matrix and the
  // look-ahead keeps it beside the next diagonal block.
  const bool two = P >= kTwoLevelMinPanels;
  auto bend_of = [&](int q) { return two ? std::min(P - 1, (q / NBO) * NBO + NBO - 1) : P - 1; };
  const size_t lds_tile = kTileLdsQuarter;
  for (int p = 0; p <= P; ++p) {
    const int bend_prev = p > 0 ? bend_of(p - 1) : 0;
    const int nu2 = p > 0 ? u2_tiles(P, p - 1, bend_prev) : 0;
    hipLaunchKernelGGL(chol_step, dim3((unsigned)(1 + nu2)), dim3(256), 0, s, npad, n, P, p, bend_prev, w);
    KQ_LAUNCHED("chol_step");
    if (p == P) break;
    const int q = P - p - 1;
    hipLaunchKernelGGL(chol_panel, dim3((unsigned)(4 * q + 4 * (p + 1))), dim3(256), lds_tile, s, npad, P, p, w);
    KQ_LAUNCHED("chol_panel");
    const int bend = bend_of(p);
    if (p < bend) {
      hipLaunchKernelGGL(chol_u1, dim3((unsigned)(4 * q)), dim3(256), lds_tile, s, npad, p, w);
      KQ_LAUNCHED("chol_u1");
    } else if (p < P - 1) {
      // p ends its outer block b0 .. p (two-level only)
      const int b0 = p - NBO + 1, b1 = p + 1, q2 = P - b1;
      const int64_t r0 = (int64_t)b1 * NB, c1 = (int64_t)b1 * NB;
      const int nL = (int)(NBO * ((npad - r0) / 32));
      const int nY = (int)(NBO * NB * ((c1 + 1023) / 1024));
      hipLaunchKernelGGL(chol_presplit, dim3((unsigned)(nL + nY)), dim3(256), 0, s, npad, r0, c1, nL, w);
      KQ_LAUNCHED("chol_presplit");
      // whole 8 x 8 super-tiles, their count padded to a multiple of 8 (see chol_outer)
      const int T = (q2 + 7) / 8, Cs = (b1 + 7) / 8;
      const int nsup = (T * (T + 1) / 2 + T * Cs + 7) / 8 * 8;
      hipLaunchKernelGGL(chol_outer, dim3((unsigned)(nsup * 64)), dim3(256), 0, s, npad, P, b0, w);
      KQ_LAUNCHED("chol_outer");
    }
  }
  {
    const unsigned gx = (unsigned)std::min<int64_t>((n + 255) / 256, 64);
    if (n % 4 == 0 && ldr % 4 == 0 && reinterpret_cast<uintptr_t>(R) % 16 == 0) {
      const unsigned gx4 = (unsigned)std::min<int64_t>((n / 4 + 255) / 256, 64);
      hipLaunchKernelGGL(chol_flip4, dim3(gx4, (unsigned)n), dim3(256), 0, s, n, npad, R, ldr, w);
    } else {
      hipLaunchKernelGGL(chol_flip, dim3(gx, (unsigned)n), dim3(256), 0, s, n, npad, R, ldr, w);
    }
    KQ_LAUNCHED("chol_flip");
  }
  long long h_info = -1;
  int h_flag = 0, h_nonfinite = 0;
  KQ_HIP(hipMemcpyAsync(&h_info, w.info, sizeof(h_info), hipMemcpyDeviceToHost, s));
  KQ_HIP(hipMemcpyAsync(&h_flag, w.flag, sizeof(h_flag), hipMemcpyDeviceToHost, s));
  KQ_HIP(hipMemcpyAsync(&h_nonfinite, w.nonfinite, sizeof(h_nonfinite), hipMemcpyDeviceToHost, s));
  KQ_HIP(hipStreamSynchronize(s));
  if (h_nonfinite) {
    *info = -1;
    return fail(KRONQ_ENUMERIC, "kronq_chol_inv: H holds a NaN or an infinity (or its damping term "
                "is not finite)");
  }
  if (h_flag) {
    *info = h_info;
    return fail(KRONQ_ENOTPD, "kronq_chol_inv: trailing block at processing index %lld is not "
                "positive definite", h_info);
  }
  *info = -1;
  return KRONQ_OK;
}

}  // namespace kronq
