// Kronecker factors H = scale * A^T A + beta * H on the gfx950 matrix cores.
//
// The factor H_X = E[x x^T] (and H_G = E[g g^T]) of the K-FAC Hessian
// (hyper.ai summary of the KronQ paper, Method) is a symmetric rank-N update:
// a dense contraction over the N token rows of A (N x d, row-major).  Only the
// upper-triangle tiles are computed; each is written to both triangles.
//
// bf16 path: macro tile 256 x 256, four waves (2 x 2), each wave owning a
// 128 x 128 block as 4 x 4 accumulators of v_mfma_f32_32x32x16_bf16 (bf16
// products are exact in fp32, accumulation fp32).  The contraction index is the
// token, which is the row index of A, so a lane's MFMA operand (8 consecutive
// tokens of one feature) is strided in memory: each thread loads an 8-token x
// 8-feature sub-block with eight coalesced 16-byte row loads, transposes it in
// registers (v_perm_b32), and stores 8 feature rows of 8 tokens into LDS, where
// a single ds_read_b128 then yields the operand.  K is staged 64 tokens at a
// time, double-buffered (2 x 72 KiB LDS, one workgroup per CU).
//
// fp32 path (fp32 inputs): macro tile 128 x 128 on v_mfma_f32_32x32x2f32,
// whose operands take one value per lane, so tiles are staged untransposed.
//
// Scheduling: work items are (tile, token split).  The split count S is chosen
// so that the item count nearly fills a multiple of the 256 CUs; with S > 1
// every item writes its partial tile to the workspace and a finalize kernel
// sums the splits, applies scale/beta and mirrors.  Items are numbered split-
// major over a 4 x 4 super-tile order of the upper triangle and dealt to the
// eight XCDs in contiguous ranges (workgroup b runs on XCD b % 8), so the
// workgroups that share an XCD's L2 at the same time work on the same token
// range and neighbouring tiles.
#include "kronq_internal.h"

namespace kronq {
namespace {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16_t __attribute__((__vector_size__(16 * sizeof(float))));
typedef float f32x4_t __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4_t __attribute__((__vector_size__(4 * sizeof(uint32_t))));

constexpr int kXcds = 8;
constexpr int kCUs = 256;

// ---------------- bf16 tile geometry ----------------
constexpr int BT = 256;          // macro tile edge (features)
constexpr int BK = 64;           // tokens per LDS stage
constexpr int LDK = BK + 8;      // padded LDS row (bf16 elements) = 144 bytes
constexpr int PANEL = BT * LDK;  // one panel (256 features x 64 tokens), bf16 elements
constexpr int BTHREADS = 256;

// ---------------- fp32 tile geometry ----------------
constexpr int FT = 128;
constexpr int FK = 32;
constexpr int FLD = FT + 4;      // padded LDS row (floats)
constexpr int FPANEL = FK * FLD;

struct GramParams {
  const void* A;
  int64_t N, d, lda, ldh;
  float* H;
  float* part;       // S > 1: partial tiles [item][tile][tile]
  float scale, beta;
  int T;             // tiles per side
  int ntiles;        // upper-triangle tiles
  int S;             // token splits
  int nitems;        // ntiles * S
  int per_xcd;       // ceil(nitems / 8)
  int64_t nstages;   // ceil(N / stage)
};

// Upper-triangle tile number t -> (ti, tj), tj >= ti, in 4 x 4 super-tile order.
__device__ inline void tile_coords(int t, int T, int& ti, int& tj) {
  const int SB = 4;
  const int R = (T + SB - 1) / SB;
  for (int sr = 0; sr < R; ++sr) {
    const int r0 = sr * SB, nr = min(SB, T - r0);
    for (int sc = sr; sc < R; ++sc) {
      const int c0 = sc * SB, nc = min(SB, T - c0);
      const int cnt = (sc == sr) ? nr * (nr + 1) / 2 : nr * nc;
      if (t < cnt) {
        if (sc == sr) {
          int a = 0;
          while (t >= nr - a) { t -= nr - a; ++a; }
          ti = r0 + a;
          tj = r0 + a + t;
        } else {
          ti = r0 + t / nc;
          tj = c0 + t % nc;
        }
        return;
      }
      t -= cnt;
    }
  }
  ti = tj = 0;
}

// XCD-aware item of this workgroup; false when the slot is past the end.
__device__ inline bool my_item(const GramParams& p, int& item) {
  const int b = blockIdx.x;
  item = (b % kXcds) * p.per_xcd + b / kXcds;
  return (b / kXcds) < p.per_xcd && item < p.nitems;
}

__device__ inline void split_range(const GramParams& p, int s, int64_t& st0, int64_t& st1) {
  st0 = p.nstages * s / p.S;
  st1 = p.nstages * (s + 1) / p.S;
}

// Store one accumulator element pair (i, j) and its mirror.
__device__ inline void put(const GramParams& p, int64_t i, int64_t j, float v, bool mirror) {
  if (i >= p.d || j >= p.d) return;
  float* h = p.H + i * p.ldh + j;
  *h = (p.beta != 0.0f) ? fmaf(p.scale, v, p.beta * *h) : p.scale * v;
  if (mirror) {
    float* g = p.H + j * p.ldh + i;
    *g = (p.beta != 0.0f) ? fmaf(p.scale, v, p.beta * *g) : p.scale * v;
  }
}

// =====================================================================
// bf16 kernel
// =====================================================================

// Load the 8 x 8 (token x feature) sub-block of this thread into registers.
// kAnyD: d need not be a multiple of 8 (element-wise tail); otherwise a whole
// 8-feature group is either inside or outside d and rows past N read zeros.
template <bool kAnyD>
__device__ inline void load_sub(const uint16_t* __restrict__ A, int64_t lda, int64_t N, int64_t d,
                                int64_t row0, int64_t col0, u32x4_t (&v)[8]) {
  if (!kAnyD) {
    const bool col_ok = col0 < d;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int64_t row = row0 + r;
      const bool ok = col_ok && row < N;
      const int64_t rr = ok ? row : 0, cc = ok ? col0 : 0;
      u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(A + rr * lda + cc));
      v[r] = ok ? x : u32x4_t{0u, 0u, 0u, 0u};
    }
  } else {
    for (int r = 0; r < 8; ++r) {
      const int64_t row = row0 + r;
      uint32_t w[4] = {0u, 0u, 0u, 0u};
      if (row < N) {
        for (int c = 0; c < 8; ++c)
          if (col0 + c < d) w[c >> 1] |= (uint32_t)A[row * lda + col0 + c] << (16 * (c & 1));
      }
      v[r] = u32x4_t{w[0], w[1], w[2], w[3]};
    }
  }
}

// Transpose the 8 x 8 block of 16-bit values and store 8 feature rows.
__device__ inline void store_sub(uint16_t* __restrict__ P, int fb, int tb, const u32x4_t (&v)[8]) {
  // v[r][q] holds features 2q (low half) and 2q + 1 (high half) of token r
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
    const int q = c >> 1;
    u32x4_t o;
    o[0] = __builtin_amdgcn_perm(v[1][q], v[0][q], sel);
    o[1] = __builtin_amdgcn_perm(v[3][q], v[2][q], sel);
    o[2] = __builtin_amdgcn_perm(v[5][q], v[4][q], sel);
    o[3] = __builtin_amdgcn_perm(v[7][q], v[6][q], sel);
    *reinterpret_cast<u32x4_t*>(P + (8 * fb + c) * LDK + 8 * tb) = o;
  }
}

template <bool kAnyD>
__global__ void __launch_bounds__(BTHREADS, 1) gram_bf16_kernel(GramParams p) {
  int item;
  if (!my_item(p, item)) return;
  const int s = item / p.ntiles;
  const int t = item % p.ntiles;
  int ti, tj;
  tile_coords(t, p.T, ti, tj);
  const bool diag = (ti == tj);
  const int64_t I0 = (int64_t)ti * BT, J0 = (int64_t)tj * BT;
  int64_t st0, st1;
  split_range(p, s, st0, st1);

  extern __shared__ __align__(16) uint16_t lds[];
  // buffer b holds panel I at lds + 2 b PANEL and panel J right after it

  const int tid = threadIdx.x;
  const int tb = tid & 7, fb = tid >> 3;  // sub-block of this thread
  const uint16_t* A = static_cast<const uint16_t*>(p.A);

  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lk = lane >> 5;

  f32x16_t acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;

  u32x4_t ri[8], rj[8];
  auto gload = [&](int64_t st) {
    const int64_t row0 = st * BK + 8 * tb;
    load_sub<kAnyD>(A, p.lda, p.N, p.d, row0, I0 + 8 * fb, ri);
    if (!diag) load_sub<kAnyD>(A, p.lda, p.N, p.d, row0, J0 + 8 * fb, rj);
  };
  auto lstore = [&](int buf) {
    store_sub(lds + 2 * buf * PANEL, fb, tb, ri);
    if (!diag) store_sub(lds + (2 * buf + 1) * PANEL, fb, tb, rj);
  };

  gload(st0);
  lstore(0);
  __syncthreads();

  int buf = 0;
  for (int64_t st = st0; st < st1; ++st) {
    const bool more = (st + 1 < st1);
    if (more) gload(st + 1);
    const uint16_t* PI = lds + 2 * buf * PANEL;
    const uint16_t* PJ = diag ? PI : PI + PANEL;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8_t af[4], bfr[4];
#pragma unroll
      for (int a = 0; a < 4; ++a)
        af[a] = *reinterpret_cast<const bf16x8_t*>(PI + (wm * 128 + 32 * a + lr) * LDK + 16 * kk + 8 * lk);
#pragma unroll
      for (int b = 0; b < 4; ++b)
        bfr[b] = *reinterpret_cast<const bf16x8_t*>(PJ + (wn * 128 + 32 * b + lr) * LDK + 16 * kk + 8 * lk);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bfr[b], acc[a][b], 0, 0, 0);
    }
    if (more) lstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

  // epilogue.  32x32 accumulator layout: lane holds column lr; register v holds
  // row 8 * (v / 4) + 4 * lk + (v % 4).
  if (p.S == 1) {
    const int64_t ib = I0 + wm * 128 + 4 * lk, jb = J0 + wn * 128 + lr;
    const bool beta0 = (p.beta == 0.0f);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t i = ib + 32 * a + 8 * (v >> 2) + (v & 3);
          const int64_t j = jb + 32 * b;
          if (i < p.d && j < p.d) {
            const float x = p.scale * acc[a][b][v];
            float* h = p.H + i * p.ldh + j;
            *h = beta0 ? x : fmaf(p.beta, *h, x);
            if (!diag) {
              float* g = p.H + j * p.ldh + i;
              *g = beta0 ? x : fmaf(p.beta, *g, x);
            }
          }
        }
  } else {
    float* out = p.part + (int64_t)item * BT * BT + (wm * 128 + 4 * lk) * BT + wn * 128 + lr;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          __builtin_nontemporal_store(acc[a][b][v],
                                      out + (32 * a + 8 * (v >> 2) + (v & 3)) * BT + 32 * b);
  }
}

// =====================================================================
// fp32 kernel
// =====================================================================

__global__ void __launch_bounds__(256, 2) gram_f32_kernel(GramParams p) {
  int item;
  if (!my_item(p, item)) return;
  const int s = item / p.ntiles;
  const int t = item % p.ntiles;
  int ti, tj;
  tile_coords(t, p.T, ti, tj);
  const bool diag = (ti == tj);
  const int64_t I0 = (int64_t)ti * FT, J0 = (int64_t)tj * FT;
  int64_t st0, st1;
  split_range(p, s, st0, st1);

  extern __shared__ __align__(16) float fl[];
  const float* A = static_cast<const float*>(p.A);

  const int tid = threadIdx.x;
  const int c4 = tid & 31, r0 = tid >> 5;  // float4 column, first row
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lk = lane >> 5;

  f32x16_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;

  float4 ri[4], rj[4];
  auto ld4 = [&](int64_t row, int64_t col) -> float4 {
    if (row >= p.N) return make_float4(0.f, 0.f, 0.f, 0.f);
    if (col + 4 <= p.d) return *reinterpret_cast<const float4*>(A + row * p.lda + col);
    float w[4];
    for (int q = 0; q < 4; ++q) w[q] = (col + q < p.d) ? A[row * p.lda + col + q] : 0.f;
    return make_float4(w[0], w[1], w[2], w[3]);
  };
  auto gload = [&](int64_t st) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t row = st * FK + r0 + 8 * q;
      ri[q] = ld4(row, I0 + 4 * c4);
      if (!diag) rj[q] = ld4(row, J0 + 4 * c4);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      *reinterpret_cast<float4*>(fl + 2 * buf * FPANEL + (r0 + 8 * q) * FLD + 4 * c4) = ri[q];
      if (!diag)
        *reinterpret_cast<float4*>(fl + (2 * buf + 1) * FPANEL + (r0 + 8 * q) * FLD + 4 * c4) = rj[q];
    }
  };

  gload(st0);
  lstore(0);
  __syncthreads();
  int buf = 0;
  for (int64_t st = st0; st < st1; ++st) {
    const bool more = (st + 1 < st1);
    if (more) gload(st + 1);
    const float* PI = fl + 2 * buf * FPANEL;
    const float* PJ = diag ? PI : PI + FPANEL;
#pragma unroll
    for (int kk = 0; kk < FK / 2; ++kk) {
      float af[2], bfv[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) af[a] = PI[(2 * kk + lk) * FLD + wm * 64 + 32 * a + lr];
#pragma unroll
      for (int b = 0; b < 2; ++b) bfv[b] = PJ[(2 * kk + lk) * FLD + wn * 64 + 32 * b + lr];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[a], bfv[b], acc[a][b], 0, 0, 0);
    }
    if (more) lstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

  if (p.S == 1) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t i = I0 + wm * 64 + 32 * a + 8 * (v >> 2) + 4 * lk + (v & 3);
          const int64_t j = J0 + wn * 64 + 32 * b + lr;
          put(p, i, j, acc[a][b][v], !diag);
        }
  } else {
    float* out = p.part + (int64_t)item * FT * FT;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = wm * 64 + 32 * a + 8 * (v >> 2) + 4 * lk + (v & 3);
          const int c = wn * 64 + 32 * b + lr;
          out[r * FT + c] = acc[a][b][v];
        }
  }
}

// Sum the S partial tiles, apply scale/beta, write both triangles.
// Grid: (tile * 64) blocks of 256 threads; each thread handles 4 columns of
// one row of the tile; TS = tile edge.
template <int TS>
__global__ void __launch_bounds__(256) gram_finalize_kernel(GramParams p) {
  constexpr int ROWS_PER_BLOCK = 256 * 4 / TS;
  const int t = blockIdx.x / (TS / ROWS_PER_BLOCK);
  const int rblk = blockIdx.x % (TS / ROWS_PER_BLOCK);
  int ti, tj;
  tile_coords(t, p.T, ti, tj);
  const bool diag = (ti == tj);
  const int r = rblk * ROWS_PER_BLOCK + threadIdx.x / (TS / 4);
  const int c = 4 * (threadIdx.x % (TS / 4));
  f32x4_t sum = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < p.S; ++s) {
    const float* src = p.part + ((int64_t)(s * p.ntiles + t) * TS + r) * TS + c;
    sum += *reinterpret_cast<const f32x4_t*>(src);
  }
  const int64_t i = (int64_t)ti * TS + r;
#pragma unroll
  for (int q = 0; q < 4; ++q) put(p, i, (int64_t)tj * TS + c + q, sum[q], !diag);
}

int choose_splits(int ntiles, int64_t nstages) {
  // smallest S whose item count fills at least 90% of whole CU rounds; else the
  // best fill; never more splits than stages
  int best = 1;
  double best_eff = 0.0;
  const int smax = (int)std::min<int64_t>(64, nstages);
  for (int S = 1; S <= smax; ++S) {
    const int64_t items = (int64_t)ntiles * S;
    const int64_t rounds = (items + kCUs - 1) / kCUs;
    const double eff = (double)items / (double)(rounds * kCUs);
    if (eff >= 0.9) return S;
    if (eff > best_eff + 1e-9) { best_eff = eff; best = S; }
  }
  return best;
}

void plan(int64_t N, int64_t d, int32_t dtype, int& T, int& ntiles, int& S, int64_t& nstages) {
  const int ts = (dtype == KRONQ_BF16) ? BT : FT;
  const int kst = (dtype == KRONQ_BF16) ? BK : FK;
  T = (int)((d + ts - 1) / ts);
  ntiles = T * (T + 1) / 2;
  nstages = (N + kst - 1) / kst;
  S = choose_splits(ntiles, nstages);
}

}  // namespace

size_t gram_ws_bytes(int64_t N, int64_t d, int32_t dtype) {
  int T, ntiles, S;
  int64_t nstages;
  plan(N, d, dtype, T, ntiles, S, nstages);
  if (S == 1) return 0;
  const int ts = (dtype == KRONQ_BF16) ? BT : FT;
  return (size_t)ntiles * (size_t)S * (size_t)ts * (size_t)ts * sizeof(float);
}

kronq_status gram_launch(const void* A, int32_t dtype, int64_t N, int64_t d, int64_t lda, float* H,
                         int64_t ldh, float scale, float beta, void* ws, size_t ws_bytes,
                         hipStream_t s) {
  (void)ws_bytes;
  GramParams p{};
  p.A = A;
  p.N = N;
  p.d = d;
  p.lda = lda;
  p.ldh = ldh;
  p.H = H;
  p.part = static_cast<float*>(ws);
  p.scale = scale;
  p.beta = beta;
  plan(N, d, dtype, p.T, p.ntiles, p.S, p.nstages);
  p.nitems = p.ntiles * p.S;
  p.per_xcd = (p.nitems + kXcds - 1) / kXcds;
  const int grid = p.per_xcd * kXcds;
  if (dtype == KRONQ_BF16) {
    const size_t lds = 4 * PANEL * sizeof(uint16_t);
    if (d % 8 == 0) {
      KQ_HIP(hipFuncSetAttribute((const void*)gram_bf16_kernel<false>,
                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
      hipLaunchKernelGGL(gram_bf16_kernel<false>, dim3(grid), dim3(BTHREADS), lds, s, p);
    } else {
      KQ_HIP(hipFuncSetAttribute((const void*)gram_bf16_kernel<true>,
                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
      hipLaunchKernelGGL(gram_bf16_kernel<true>, dim3(grid), dim3(BTHREADS), lds, s, p);
    }
    KQ_LAUNCHED("gram_bf16_kernel");
    if (p.S > 1) {
      hipLaunchKernelGGL(gram_finalize_kernel<BT>, dim3(p.ntiles * (BT / (1024 / BT))), dim3(256), 0, s, p);
      KQ_LAUNCHED("gram_finalize_kernel");
    }
  } else {
    const size_t lds = 4 * FPANEL * sizeof(float);
    hipLaunchKernelGGL(gram_f32_kernel, dim3(grid), dim3(256), lds, s, p);
    KQ_LAUNCHED("gram_f32_kernel");
    if (p.S > 1) {
      hipLaunchKernelGGL(gram_finalize_kernel<FT>, dim3(p.ntiles * (FT / (1024 / FT))), dim3(256), 0, s, p);
      KQ_LAUNCHED("gram_finalize_kernel");
    }
  }
  return KRONQ_OK;
}

}  // namespace kronq
