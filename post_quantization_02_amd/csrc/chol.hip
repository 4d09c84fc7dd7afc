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
// with A so it changes nothing):
//   diag kernel   (1 workgroup): factor A_pp in fp64 in LDS, invert it by
//                 recursive doubling, store Linv_pp (fp32); report pivots <= 0
//   panel kernel  : L_ip = A_ip Linv_pp^T (stored over A_ip) and
//                   M_ip = L_ip Linv_pp, for every row tile i > p
//   update kernel : A_ij -= L_ip L_jp^T        (i >= j > p; Cholesky SYRK)
//                   B_i[:, c] -= M_ip B_p[:, c] (i > p, c <= p; forward
//                   substitution of L Y = I with B initialised to I)
// and finally Y_p = Linv_pp B_p and R = J Y J.  All tile products run on the
// fp32 matrix cores (v_mfma_f32_32x32x2f32), 128 x 128 output tiles with four
// waves of 64 x 64.  A device flag set by a failed pivot makes every later
// kernel return at once; the host reads the flag after the last launch.
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
  float* M;       // npad x NB   (M_ip for the current panel)
  float* Linv;    // P x NB x NB (inverse diagonal blocks)
  double* damp;   // lambda * mean(diag H)
  int* flag;      // nonzero after a failed pivot
  long long* info;
};

size_t ws_layout(int64_t n, CholWs* w, void* base) {
  const int64_t npad = (n + NB - 1) / NB * NB;
  const size_t sA = align_up((size_t)npad * npad * sizeof(float), 256);
  const size_t sM = align_up((size_t)npad * NB * sizeof(float), 256);
  size_t off = 0;
  char* b = static_cast<char*>(base);
  if (w) w->A = reinterpret_cast<float*>(b + off);
  off += sA;
  if (w) w->B = reinterpret_cast<float*>(b + off);
  off += sA;
  if (w) w->M = reinterpret_cast<float*>(b + off);
  off += sM;
  if (w) w->Linv = reinterpret_cast<float*>(b + off);
  off += sM;
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

// Factor the NB x NB block A_pp (lower, fp64) and invert it; Linv_pp stored in
// fp32 (full block, zeros above the diagonal).
__global__ void __launch_bounds__(256) chol_diag(int64_t npad, int64_t n, int p, CholWs w) {
  if (*w.flag) return;
  extern __shared__ __align__(16) double sd[];
  double* a = sd;              // NB x NB
  double* col = sd + NB * NB;  // NB
  __shared__ int bad;
  const int tid = threadIdx.x;
  const float* Ap = w.A + (int64_t)p * NB * npad + (int64_t)p * NB;
  for (int e = tid; e < NB * NB; e += 256) {
    const int i = e / NB, k = e % NB;
    a[e] = (k <= i) ? (double)Ap[(int64_t)i * npad + k] : 0.0;
  }
  if (tid == 0) bad = -1;
  __syncthreads();
  for (int j = 0; j < NB; ++j) {
    if (tid < NB && tid >= j) col[tid] = a[tid * NB + j];
    __syncthreads();
    const double d = col[j];
    if (!(d > 0.0)) {
      if (tid == 0) bad = j;
      break;
    }
    const double lj = sqrt(d);
    __syncthreads();
    if (tid < NB && tid > j) {
      const double v = col[tid] / lj;
      col[tid] = v;
      a[tid * NB + j] = v;
    }
    if (tid == 0) a[j * NB + j] = lj;
    __syncthreads();
    const int cnt = NB - 1 - j;
    for (int e = tid; e < cnt * cnt; e += 256) {
      const int i = j + 1 + e / cnt, k = j + 1 + e % cnt;
      if (k <= i) a[i * NB + k] -= col[i] * col[k];
    }
    __syncthreads();
  }
  __syncthreads();
  if (bad >= 0) {
    if (tid == 0) {
      // reversed position p*NB + bad is processing index n - 1 - that
      const int64_t pos = (int64_t)p * NB + bad;
      *w.info = (pos < n) ? (long long)(n - 1 - pos) : (long long)-2;
      *w.flag = 1;
    }
    return;
  }
  // invert the lower triangle in place by recursive doubling:
  // diag 1 / l_ii, then for block size s = 2, 4, ..., NB:
  //   X21 = -X22 (L21 X11), with the product L21 X11 staged in the (unused)
  //   strictly upper block of the same diagonal block.
  for (int i = tid; i < NB; i += 256) a[i * NB + i] = 1.0 / a[i * NB + i];
  __syncthreads();
  for (int s = 2; s <= NB; s <<= 1) {
    const int h = s / 2;
    const int nblk = NB / s;
    // T = L21 X11 : (h x h) per block, stored at [o + r][o + h + c]
    for (int e = tid; e < nblk * h * h; e += 256) {
      const int blk = e / (h * h), r = (e / h) % h, c = e % h;
      const int o = blk * s;
      double t = 0.0;
      for (int k = c; k < h; ++k) t += a[(o + h + r) * NB + o + k] * a[(o + k) * NB + o + c];
      a[(o + r) * NB + o + h + c] = t;
    }
    __syncthreads();
    // X21 = -X22 T
    for (int e = tid; e < nblk * h * h; e += 256) {
      const int blk = e / (h * h), r = (e / h) % h, c = e % h;
      const int o = blk * s;
      double t = 0.0;
      for (int k = 0; k <= r; ++k) t += a[(o + h + r) * NB + o + h + k] * a[(o + k) * NB + o + h + c];
      a[(o + h + r) * NB + o + c] = -t;
    }
    __syncthreads();
  }
  float* L = w.Linv + (int64_t)p * NB * NB;
  for (int e = tid; e < NB * NB; e += 256) {
    const int i = e / NB, k = e % NB;
    L[e] = (k <= i) ? (float)a[e] : 0.f;
  }
}

// ------------------------------------------------------- tile products

// Layout of a global operand tile: element (x, k) of a 128 x K operand.
//   XK: stored row-major as [x][k] (leading dimension ld)
//   KX: stored row-major as [k][x]
enum { XK = 0, KX = 1 };

template <int LAY>
__device__ inline void stage_load(float* sT, const float* G, int64_t ld, int k0) {
  // sT[k][x], k in [0, KS), x in [0, NB)
  const int tid = threadIdx.x;
  if (LAY == XK) {
    // 128 rows x 32 k: thread reads float4 along k
#pragma unroll
    for (int q = 0; q < (NB * KS / 4) / 256; ++q) {
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
    for (int q = 0; q < (NB * KS / 4) / 256; ++q) {
      const int idx = tid + 256 * q;
      const int k = idx >> 5, x4 = (idx & 31) * 4;
      const float4 v = *reinterpret_cast<const float4*>(G + (int64_t)(k0 + k) * ld + x4);
      sT[k * LDT + x4 + 0] = v.x;
      sT[k * LDT + x4 + 1] = v.y;
      sT[k * LDT + x4 + 2] = v.z;
      sT[k * LDT + x4 + 3] = v.w;
    }
  }
}

// acc (per wave 64 x 64 of the 128 x 128 result) = sum_k A(x=i, k) B(x=j, k)
template <int LA, int LB>
__device__ inline void tile_mma(f32x16_t (&acc)[2][2], const float* Ag, int64_t lda, const float* Bg,
                                int64_t ldb, int K, float* sA, float* sB) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lk = lane >> 5;
  for (int k0 = 0; k0 < K; k0 += KS) {
    __syncthreads();
    stage_load<LA>(sA, Ag, lda, k0);
    stage_load<LB>(sB, Bg, ldb, k0);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < KS; kk += 2) {
      float af[2], bf[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) af[a] = sA[(kk + lk) * LDT + wm * 64 + 32 * a + lr];
#pragma unroll
      for (int b = 0; b < 2; ++b) bf[b] = sB[(kk + lk) * LDT + wn * 64 + 32 * b + lr];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[a], bf[b], acc[a][b], 0, 0, 0);
    }
  }
}

__device__ inline void zero_acc(f32x16_t (&acc)[2][2]) {
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;
}

// mode 0: C = acc; mode 1: C -= acc
template <int MODE>
__device__ inline void tile_store(float* C, int64_t ldc, const f32x16_t (&acc)[2][2]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lk = lane >> 5;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wm * 64 + 32 * a + 8 * (v >> 2) + 4 * lk + (v & 3);
        const int c = wn * 64 + 32 * b + lr;
        float* dst = C + (int64_t)r * ldc + c;
        if (MODE == 0) *dst = acc[a][b][v];
        else *dst -= acc[a][b][v];
      }
}

// L_ip = A_ip Linv^T -> A_ip ; M_ip = L_ip Linv -> M[i]
__global__ void __launch_bounds__(256) chol_panel(int64_t npad, int p, CholWs w) {
  if (*w.flag) return;
  extern __shared__ __align__(16) float sm[];
  float* sA = sm;
  float* sB = sm + KS * LDT;
  const int i = p + 1 + blockIdx.x;
  float* Aip = w.A + (int64_t)i * NB * npad + (int64_t)p * NB;
  const float* Lv = w.Linv + (int64_t)p * NB * NB;
  f32x16_t acc[2][2];
  zero_acc(acc);
  tile_mma<XK, XK>(acc, Aip, npad, Lv, NB, NB, sA, sB);  // B(j, k) = Linv[j][k]
  __syncthreads();
  tile_store<0>(Aip, npad, acc);
  // the tile is read back below by other waves of this workgroup
  __threadfence();
  __syncthreads();
  __threadfence();
  zero_acc(acc);
  tile_mma<XK, KX>(acc, Aip, npad, Lv, NB, NB, sA, sB);  // B(j, k) = Linv[k][j]
  tile_store<0>(w.M + (int64_t)i * NB * NB, NB, acc);
}

// SYRK tiles (i >= j > p) then B-update tiles (i > p, c <= p)
__global__ void __launch_bounds__(256) chol_update(int64_t npad, int P, int p, CholWs w) {
  if (*w.flag) return;
  extern __shared__ __align__(16) float sm[];
  float* sA = sm;
  float* sB = sm + KS * LDT;
  const int q = P - p - 1;             // row tiles below the panel
  const int nsyrk = q * (q + 1) / 2;
  int t = blockIdx.x;
  f32x16_t acc[2][2];
  zero_acc(acc);
  if (t < nsyrk) {
    int a = 0;
    while (t >= a + 1) { t -= a + 1; ++a; }
    const int i = p + 1 + a, j = p + 1 + t;   // j <= i
    const float* Li = w.A + (int64_t)i * NB * npad + (int64_t)p * NB;
    const float* Lj = w.A + (int64_t)j * NB * npad + (int64_t)p * NB;
    tile_mma<XK, XK>(acc, Li, npad, Lj, npad, NB, sA, sB);
    tile_store<1>(w.A + (int64_t)i * NB * npad + (int64_t)j * NB, npad, acc);
  } else {
    t -= nsyrk;
    const int i = p + 1 + t / (p + 1), c = t % (p + 1);
    const float* Mi = w.M + (int64_t)i * NB * NB;
    const float* Bp = w.B + (int64_t)p * NB * npad + (int64_t)c * NB;
    tile_mma<XK, KX>(acc, Mi, NB, Bp, npad, NB, sA, sB);
    tile_store<1>(w.B + (int64_t)i * NB * npad + (int64_t)c * NB, npad, acc);
  }
}

// Y_p[:, c] = Linv_pp B_p[:, c] in place, for all p and c <= p.
__global__ void __launch_bounds__(256) chol_finish_y(int64_t npad, CholWs w) {
  if (*w.flag) return;
  extern __shared__ __align__(16) float sm[];
  float* sA = sm;
  float* sB = sm + KS * LDT;
  int t = blockIdx.x, p = 0;
  while (t >= p + 1) { t -= p + 1; ++p; }
  const int c = t;
  float* Bt = w.B + (int64_t)p * NB * npad + (int64_t)c * NB;
  const float* Lv = w.Linv + (int64_t)p * NB * NB;
  f32x16_t acc[2][2];
  zero_acc(acc);
  tile_mma<XK, KX>(acc, Lv, NB, Bt, npad, NB, sA, sB);
  __syncthreads();
  tile_store<0>(Bt, npad, acc);
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
  const size_t lds_diag = (size_t)(NB * NB + NB) * sizeof(double);
  const size_t lds_tile = 2 * (size_t)KS * LDT * sizeof(float);
  KQ_HIP(hipFuncSetAttribute((const void*)chol_diag, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)lds_diag));
  for (int p = 0; p < P; ++p) {
    hipLaunchKernelGGL(chol_diag, dim3(1), dim3(256), lds_diag, s, npad, n, p, w);
    KQ_LAUNCHED("chol_diag");
    const int q = P - p - 1;
    if (q == 0) break;
    hipLaunchKernelGGL(chol_panel, dim3(q), dim3(256), lds_tile, s, npad, p, w);
    KQ_LAUNCHED("chol_panel");
    const int tiles = q * (q + 1) / 2 + q * (p + 1);
    hipLaunchKernelGGL(chol_update, dim3(tiles), dim3(256), lds_tile, s, npad, P, p, w);
    KQ_LAUNCHED("chol_update");
  }
  hipLaunchKernelGGL(chol_finish_y, dim3(P * (P + 1) / 2), dim3(256), lds_tile, s, npad, w);
  KQ_LAUNCHED("chol_finish_y");
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
