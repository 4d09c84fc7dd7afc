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
  const void* B;     // J panels: A for the Gram; the second operand of a cross product
  int64_t N, d, lda, ldh;
  float* H;
  const float* sub;  // cross product: subtracted after scaling (may be NULL)
  int64_t ldsub;
  bool cross;        // H = scale A^T B - sub over all tiles, no mirroring
  float* part;       // S > 1: partial tiles [item][tile][tile]
  float scale, beta;
  int T;             // tiles per side
  int ntiles;        // upper-triangle tiles
  int S;             // token splits
  int nitems;        // ntiles * S
  int per_xcd;       // ceil(nitems / 8)
  int64_t nstages;   // ceil(N / stage)
  bool vec_h;        // H 16-byte aligned and ldh a multiple of 4
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

// All-tiles number t -> (ti, tj) of a cross product, in 4 x 4 super-tile order.
__device__ inline void tile_coords_full(int t, int T, int& ti, int& tj) {
  const int SB = 4;
  const int R = (T + SB - 1) / SB;
  for (int sr = 0; sr < R; ++sr) {
    const int r0 = sr * SB, nr = min(SB, T - r0);
    const int cnt = nr * T;
    if (t < cnt) {
      const int sc = (t / nr) / SB;                    // column super-tile
      const int c0 = sc * SB, nc = min(SB, T - c0);
      const int u = t - nr * c0;                        // index inside the super-tile
      ti = r0 + u / nc;
      tj = c0 + u % nc;
      return;
    }
    t -= cnt;
  }
  ti = tj = 0;
}

__device__ inline void tile_of(const GramParams& p, int t, int& ti, int& tj) {
  if (p.cross) tile_coords_full(t, p.T, ti, tj);
  else tile_coords(t, p.T, ti, tj);
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
  float x = (p.beta != 0.0f) ? fmaf(p.scale, v, p.beta * *h) : p.scale * v;
  if (p.sub) x -= p.sub[i * p.ldsub + j];
  *h = x;
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
// bf16 kernel, direct-to-LDS pipeline (d a multiple of 256)
// =====================================================================
//
// Stage = 32 tokens of the I and J panels (256 features each), fetched with
// global_load_lds (16 bytes per lane, no register staging) into a ring of D
// LDS stages, so D - 1 stages of loads are in flight while one is consumed.
// A panel stage is stored token-major (512-byte rows, as in memory) with its
// 16-byte chunks XOR-swizzled by the token (chunk ^ SWZ[token % 4]); the MFMA
// operands (8 consecutive tokens of one feature per lane) are read with the
// transposing ds_read_b64_tr_b16: within each 16 lanes, lane j addresses token
// t0 + j / 4, features f0 + 4 (j % 4) .. + 3, and lane i receives tokens
// t0 .. t0 + 3 of feature f0 + i.  The swizzle keeps these reads free of bank
// conflicts for 32 or 64 LDS banks.

constexpr int V2K = 32;                    // tokens per stage
#ifndef KRONQ_GRAM_RING
#define KRONQ_GRAM_RING 4
#endif
constexpr int V2D = KRONQ_GRAM_RING;       // stages in the ring
constexpr int V2ROW = BT * 2;              // bytes per token row of a panel
constexpr int V2PANEL = V2K * V2ROW;       // bytes per panel stage (16 KiB)

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

// chunk swizzle {0, 6, 12, 10}[token % 4]: within any 4 consecutive tokens the
// swizzled chunk pairs are distinct mod 8 and the chunk quads distinct mod 16
__device__ __forceinline__ int v2_swz(int token) { return (0xAC60 >> (4 * (token & 3))) & 15; }

// Ring slots: each stage slot (panels I and J) is a distinct LDS object, so
// that the compiler's LDS-DMA tracking (which follows at most eight objects)
// sees that refilling one slot does not alias reads of another; otherwise
// every operand read would wait for all loads in flight.  Diagonal tiles load
// their panel into both halves.
// (Namespace-scope objects: a static local of the template below would be a
// separate object in every instantiation.)
struct V2Slot {
  unsigned char b[2][V2PANEL];
};
__shared__ __align__(16) V2Slot v2_s0, v2_s1, v2_s2, v2_s3, v2_s4;

template <int SLOT, int PN>
__device__ __forceinline__ unsigned char* v2_panel() {
  static_assert(SLOT < V2D && V2D <= 5, "ring slot");
  if constexpr (SLOT == 0) return v2_s0.b[PN];
  else if constexpr (SLOT == 1) return v2_s1.b[PN];
  else if constexpr (SLOT == 2) return v2_s2.b[PN];
  else if constexpr (SLOT == 3) return v2_s3.b[PN];
  else return v2_s4.b[PN];
}

// Per-lane state of the pipelined kernel.  Everything that depends on the
// lane is computed once: the operand read offsets (the swizzle of a lane's
// tokens is fixed because stage and half offsets are multiples of 4 tokens)
// and the byte offsets of the lane's direct loads within a stage.
struct V2Ctx {
  const GramParams* p;
  const unsigned char* gI;   // byte address of X[0][I0]
  const unsigned char* gJ;   // byte address of X[0][J0]
  int64_t row_bytes;         // lda * 2
  int rdI[4], rdJ[4];        // LDS byte offsets of the operand reads (token 0 of the half)
  int ldoff[4];              // byte offset of load q within a stage (token row * row_bytes + chunk)
  int wave, lane;
};

// An empty register-only asm hides the value of `x` from the optimizer, so the
// panel-base additions below are redone at each use instead of being hoisted
// out of the loop into one live register per (slot, panel, operand).
__device__ __forceinline__ int v2_opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Stages here are always whole (the host hands a token tail shorter than a
// stage to the generic kernel), so a load is a uniform base plus the lane's
// fixed 32-bit offset.
// The lane offset is added as an unsigned 32-bit value (it is below 2^32: a
// row within the stage times the row pitch), so each load takes the form with a
// scalar 64-bit base and a 32-bit vector offset.  Added as a signed value it
// was sign-extended into a 64-bit vector address, three VALU instructions per
// load between the MFMAs whose results landed in registers that the MFMAs just
// issued were still reading (the d = 28672 call: 190 ms that way, 182 ms this
// way, results identical).
template <int SLOT, int PN>
__device__ __forceinline__ void v2_issue_panel(const V2Ctx& c, int64_t tok0) {
  unsigned char* lbase = v2_panel<SLOT, PN>() + c.wave * 4 * 2 * V2ROW;
  const unsigned char* gbase = (PN ? c.gJ : c.gI) + tok0 * c.row_bytes;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    __builtin_amdgcn_global_load_lds((const void*)(gbase + (uint32_t)v2_opaque(c.ldoff[q])),
                                     (lds_void_t*)(lbase + q * 2 * V2ROW), 16, 0, 0);
}

template <int SLOT>
__device__ __forceinline__ void v2_issue(const V2Ctx& c, int64_t st) {
  v2_issue_panel<SLOT, 0>(c, st * V2K);
  v2_issue_panel<SLOT, 1>(c, st * V2K);
}

// tokens 0..3 and 4..7 of one feature -> the 8-value MFMA operand
__device__ __forceinline__ bf16x8_t v2_cat(i16x4_t lo, i16x4_t hi) {
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ i16x4_t v2_ld(const unsigned char* ptr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)ptr);
}

// operands of one 16-token half (HALF = 0, 1) of the stage in slot SLOT
struct V2Half {
  bf16x8_t a[4], b[4];
};

template <int SLOT, int HALF>
__device__ __forceinline__ void v2_read(const V2Ctx& c, V2Half& f) {
  const unsigned char* PI = v2_panel<SLOT, 0>() + HALF * 16 * V2ROW;
  const unsigned char* PJ = v2_panel<SLOT, 1>() + HALF * 16 * V2ROW;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const unsigned char* q = PI + v2_opaque(c.rdI[a]);
    f.a[a] = v2_cat(v2_ld(q), v2_ld(q + 4 * V2ROW));
  }
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const unsigned char* q = PJ + v2_opaque(c.rdJ[b]);
    f.b[b] = v2_cat(v2_ld(q), v2_ld(q + 4 * V2ROW));
  }
}

__device__ __forceinline__ void v2_mma(const V2Half& f, f32x16_t (&acc)[4][4]) {
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
      acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[a], f.b[b], acc[a][b], 0, 0, 0);
}

// interleave the 16 MFMAs of a half-stage with the 16 operand reads of the
// next half: two reads after each of the first eight MFMAs, so that the last
// read has landed well before the next half's first MFMA waits for it
__device__ __forceinline__ void v2_interleave() {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);    // eight MFMAs
}

// s_waitcnt immediate: at most `vm` loads in flight (vmcnt, 6 bits split over
// [3:0] and [15:14]), expcnt unconstrained, at most `lgkm` LDS operations
constexpr int v2_cnt(int vm, int lgkm) { return (vm & 15) | (7 << 4) | (lgkm << 8) | ((vm >> 4) << 14); }

// Wait until stage it + 1 of this wave's loads has landed (8 loads per stage;
// stages it + 2 .. it + D - 1 stay in flight) and every LDS read of this wave has
// returned, so that the barrier which follows orders all reads of slot K
// before its refill.  Every step issues exactly one stage, so the count is
// the same at every step.
__device__ __forceinline__ void v2_wait_next() { __builtin_amdgcn_s_waitcnt(v2_cnt(8 * (V2D - 2), 0)); }

// Step `it` with slot K = it mod D.  On entry H0 holds the first half of
// stage it.  First half: multiply H0 while reading the second half into H1.
// Then wait for stage it + 1 and synchronize (every wave has finished reading
// slot K), refill slot K with stage it + D, and multiply H1 while reading the
// first half of stage it + 1 into H0.
//
// The step has no branch.  Past the end of the split the refill loads the
// split's last stage again (in bounds, never consumed), and after the last
// stage the read of "stage it + 1" fetches LDS data that is never used.  A
// conditional refill would leave a control-flow join after which the
// compiler can no longer tell which ring slot a load writes, and it would then
// make every operand read wait for all loads in flight; conditional multiplies
// would merge the accumulators at a join.
template <int K>
__device__ __forceinline__ void v2_step(const V2Ctx& c, int64_t it, int64_t st0, int64_t st_last,
                                        V2Half& H0, V2Half& H1, f32x16_t (&acc)[4][4]) {
  v2_read<K, 1>(c, H1);
  v2_mma(H0, acc);
  v2_interleave();
  v2_wait_next();
  __builtin_amdgcn_s_barrier();
  v2_issue<K>(c, min<int64_t>(st0 + it + V2D, st_last));
  v2_read<(K + 1) % V2D, 0>(c, H0);
  v2_mma(H1, acc);
  v2_interleave();
}

// Item of a pipelined-kernel workgroup.  The split-major item list (item =
// s * ntiles + t, tiles in super-tile order) is cut into groups of 32
// consecutive items, and group k runs on XCD k % 8 (workgroup b runs on XCD
// b % 8): the 32 workgroups of an XCD stream one token range over a compact
// range of tiles that share most of their panels in its L2, and the XCDs
// stream at most a few token ranges at a time, so the memory-side cache
// serves the panels that several XCDs read.
__device__ inline bool my_item_group(const GramParams& p, int& item) {
  const int b = blockIdx.x;
  const int x = b % kXcds, j = b / kXcds;
  const int it = 32 * (kXcds * (j / 32) + x) + j % 32;
  if (it >= p.nitems) return false;
  item = it;
  return true;
}

// Lockstep of the 32 workgroups of an XCD (one split, S = 1).  With a single
// split an item streams all N tokens (thousands of stages), and workgroups
// that started together drift apart by more than the few stages of their
// shared panels that fit the XCD's L2, so the panels came from the fabric
// again for nearly every tile.  The persistent variant therefore meets at a
// barrier of its XCD group every kSyncStages stages: an agent-scope counter per
// XCD that each workgroup increments and then polls until every workgroup of
// the group has arrived.  The barrier only orders timing (no data passes
// through it), and the poll is bounded: after kSyncSpins polls a workgroup
// goes on, so a group member that is not resident can delay the others but
// never stop them.
constexpr int kSyncStages = 128;
constexpr int kSyncSpins = 4096;
constexpr int kSyncStride = 64;   // counters 256 bytes apart

struct GramSync {
  unsigned* ctr;       // this XCD's counter (NULL: no lockstep)
  unsigned target;     // counter value once the group has reached this barrier
  unsigned act;        // workgroups in the current group
};

__device__ __forceinline__ void xcd_barrier(GramSync& sy) {
  sy.target += sy.act;
  __builtin_amdgcn_s_barrier();
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(sy.ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int k = 0; k < kSyncSpins; ++k) {
      if (__hip_atomic_load(sy.ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= sy.target) break;
      __builtin_amdgcn_s_sleep(8);
    }
  }
  __builtin_amdgcn_s_barrier();
}

__global__ void gram_sync_clear(unsigned* ctr) {
  if (threadIdx.x < kXcds) ctr[threadIdx.x * kSyncStride] = 0u;
}

template <bool SYNC>
__device__ __forceinline__ void gram_lds_item(const GramParams& p, int item, GramSync& sy) {
  const int s = item / p.ntiles;
  const int t = item % p.ntiles;
  int ti, tj;
  tile_of(p, t, ti, tj);
  const int64_t I0 = (int64_t)ti * BT, J0 = (int64_t)tj * BT;
  const bool diag = ti == tj;
  const int tid = threadIdx.x;
  // wave index as a uniform value, so LDS bases of the direct loads (M0) are
  // scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;

  V2Ctx c;
  c.p = &p;
  c.wave = wave;
  c.lane = lane;
  c.row_bytes = p.lda * 2;
  c.gI = static_cast<const unsigned char*>(p.A) + I0 * 2;
  c.gJ = static_cast<const unsigned char*>(p.B) + J0 * 2;
  {
    // operand reads: group g = lane / 16, j = lane % 16 addresses token
    // 8 (g / 2) + j / 4 (+ 4 for the second read) and features
    // base + 16 (g % 2) + 4 (j % 4) .. + 3
    const int g = lane >> 4, j = lane & 15;
    const int tok = 8 * (g >> 1) + (j >> 2);
    const int sw = v2_swz(tok);
    const int fo = 16 * (g & 1) + 4 * (j & 3);
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int fi = wm * 128 + 32 * a + fo, fj = wn * 128 + 32 * a + fo;
      c.rdI[a] = tok * V2ROW + (((fi >> 3) ^ sw) << 4) + (fi & 7) * 2;
      c.rdJ[a] = tok * V2ROW + (((fj >> 3) ^ sw) << 4) + (fj & 7) * 2;
    }
    // loads: row pair 4 * wave + q; lane covers token row 2 * pair + lane / 32
    // and LDS chunk lane % 32, holding logical chunk (lane % 32) ^ swz(row)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = 2 * (4 * wave + q) + (lane >> 5);
      const int lchunk = (lane & 31) ^ v2_swz(row);
      c.ldoff[q] = (int)(row * c.row_bytes) + lchunk * 16;
    }
  }
  (void)diag;
  // token range of this split: whole units of V2D stages (N is a multiple of
  // V2D * V2K tokens and the unit count is at least S)
  const int64_t nunits = p.N / (V2D * V2K);
  const int64_t u0 = nunits * s / p.S, u1 = nunits * (s + 1) / p.S;
  const int64_t st0 = V2D * u0, nstages = V2D * (u1 - u0);
  const int64_t st_last = st0 + nstages - 1;

  f32x16_t acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;

  V2Half H0, H1;
  v2_issue<0>(c, st0);
  v2_issue<1>(c, st0 + 1);
  v2_issue<2>(c, st0 + 2);
  v2_issue<3>(c, st0 + 3);
  if constexpr (V2D > 4) v2_issue<V2D - 1>(c, st0 + V2D - 1);
  __builtin_amdgcn_s_waitcnt(v2_cnt(8 * (V2D - 1), 0));  // stage 0 landed
  __builtin_amdgcn_s_barrier();
  v2_read<0, 0>(c, H0);
  for (int64_t it = 0; it < nstages; it += V2D) {
    v2_step<0>(c, it, st0, st_last, H0, H1, acc);
    v2_step<1>(c, it + 1, st0, st_last, H0, H1, acc);
    v2_step<2>(c, it + 2, st0, st_last, H0, H1, acc);
    v2_step<3>(c, it + 3, st0, st_last, H0, H1, acc);
    if constexpr (V2D > 4) v2_step<V2D - 1>(c, it + V2D - 1, st0, st_last, H0, H1, acc);
    if constexpr (SYNC) {
      if ((it + V2D) % kSyncStages == 0 && it + V2D < nstages) xcd_barrier(sy);
    }
  }
  // the refills past the end are still landing in LDS: drain them before the
  // workgroup can exit
  __builtin_amdgcn_s_waitcnt(v2_cnt(0, 0));

  const int lr = lane & 31, lk = lane >> 5;
  if (p.S == 1) {
    const int64_t ib = I0 + wm * 128 + 4 * lk, jb = J0 + wn * 128 + lr;
    const bool beta0 = (p.beta == 0.0f);
    const bool mirror = !diag && !p.cross;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t i = ib + 32 * a + 8 * (v >> 2) + (v & 3);
          const int64_t jj = jb + 32 * b;
          const float x = p.scale * acc[a][b][v];
          float* h = p.H + i * p.ldh + jj;
          if (p.sub) *h = (beta0 ? x : fmaf(p.beta, *h, x)) - p.sub[i * p.ldsub + jj];
          else *h = beta0 ? x : fmaf(p.beta, *h, x);
          if (mirror) {
            float* gg = p.H + jj * p.ldh + i;
            *gg = beta0 ? x : fmaf(p.beta, *gg, x);
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

__global__ void __launch_bounds__(BTHREADS, 1) gram_bf16_lds_kernel(GramParams p) {
  int item;
  if (!my_item_group(p, item)) return;
  GramSync sy{nullptr, 0u, 0u};
  gram_lds_item<false>(p, item, sy);
}

// Persistent variant for one split: a grid of kCUs workgroups, workgroup b on
// XCD x = b % 8 in slot b / 8 of its group; round r runs item 32 (8 r + x) +
// slot (the item numbering of my_item_group), with the XCD group in lockstep.
__global__ void __launch_bounds__(BTHREADS, 1) gram_bf16_lds_sync_kernel(GramParams p, unsigned* ctr) {
  const int b = blockIdx.x;
  const int x = b % kXcds, slot = b / kXcds;
  GramSync sy{ctr + x * kSyncStride, 0u, 0u};
  for (int r = 0;; ++r) {
    const int g = kXcds * r + x;
    if (32 * g >= p.nitems) break;
    const int act = min(32, p.nitems - 32 * g);
    if (slot >= act) break;   // only the last group can be partial
    sy.act = (unsigned)act;
    gram_lds_item<true>(p, 32 * g + slot, sy);
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

// Sum the S partial tiles, apply scale/beta, write both triangles.  A
// workgroup takes a 64 x 64 sub-block of a tile as 1024 four-float vectors:
// vector f = threadIdx + 256 q is row f / 16, columns 4 (f % 16) .. + 3, so a
// wave covers four 256-byte row segments.  The splits are summed in order;
// for an off-diagonal tile the transposed copy goes through LDS, so that the
// mirrored writes are row segments too.
__device__ __forceinline__ void put4(const GramParams& p, int64_t i, int64_t j, f32x4_t v) {
  if (p.vec_h && i < p.d && j + 4 <= p.d) {   // vec_h: H (and sub) 16-byte rows
    f32x4_t* h = reinterpret_cast<f32x4_t*>(p.H + i * p.ldh + j);
    f32x4_t x;
    if (p.beta != 0.0f) {
      const f32x4_t o = *h;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = fmaf(p.scale, v[e], p.beta * o[e]);
    } else {
      x = v * p.scale;
    }
    if (p.sub) {
      const f32x4_t s4 = *reinterpret_cast<const f32x4_t*>(p.sub + i * p.ldsub + j);
      x -= s4;
    }
    *h = x;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) put(p, i, j + e, v[e], false);
  }
}

template <int TS>
__global__ void __launch_bounds__(256) gram_finalize_kernel(GramParams p) {
  constexpr int SUB = 64, NSUB = TS / SUB;
  __shared__ float tr[SUB][SUB + 1];
  const int t = blockIdx.x / (NSUB * NSUB), sb = blockIdx.x % (NSUB * NSUB);
  const int sr = sb / NSUB, sc = sb % NSUB;
  int ti, tj;
  tile_of(p, t, ti, tj);
  const bool diag = (ti == tj);
  f32x4_t sum[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) sum[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < p.S; ++k) {
    const float* src = p.part + ((int64_t)(k * p.ntiles + t) * TS + sr * SUB) * TS + sc * SUB;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int f = threadIdx.x + 256 * q, rr = f >> 4, c4 = (f & 15) * 4;
      sum[q] += *reinterpret_cast<const f32x4_t*>(src + (int64_t)rr * TS + c4);
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int f = threadIdx.x + 256 * q, rr = f >> 4, c4 = (f & 15) * 4;
    put4(p, (int64_t)ti * TS + sr * SUB + rr, (int64_t)tj * TS + sc * SUB + c4, sum[q]);
  }
  if (diag || p.cross) return;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int f = threadIdx.x + 256 * q, rr = f >> 4, c4 = (f & 15) * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) tr[rr][c4 + e] = sum[q][e];
  }
  __syncthreads();
  // mirrored: row tj * TS + sc * 64 + rr, columns ti * TS + sr * 64 + c4 ..
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int f = threadIdx.x + 256 * q, rr = f >> 4, c4 = (f & 15) * 4;
    const f32x4_t v = {tr[c4][rr], tr[c4 + 1][rr], tr[c4 + 2][rr], tr[c4 + 3][rr]};
    put4(p, (int64_t)tj * TS + sc * SUB + rr, (int64_t)ti * TS + sr * SUB + c4, v);
  }
}

int choose_splits(int ntiles, int64_t nstages) {
  // smallest S whose item count fills at least 98% of whole CU rounds, else
  // the best fill; at most 16 rounds of items (so the partial tiles stay a
  // small multiple of H) and never more splits than stages
  int best = 1;
  double best_eff = 0.0;
  const int smax = (int)std::max<int64_t>(
      1, std::min<int64_t>(std::min<int64_t>(64, nstages), 16 * kCUs / ntiles));
  for (int S = 1; S <= smax; ++S) {
    const int64_t items = (int64_t)ntiles * S;
    const int64_t rounds = (items + kCUs - 1) / kCUs;
    const double eff = (double)items / (double)(rounds * kCUs);
    if (eff >= 0.98) return S;
    if (eff > best_eff + 1e-9) { best_eff = eff; best = S; }
  }
  return best;
}

// the one-split launch of the direct-to-LDS pipeline runs persistent, its
// XCD groups in lockstep (needs the counters in the workspace)
bool sync_launch(int64_t N, int64_t d, int32_t dtype) {
  return dtype == KRONQ_BF16 && d % BT == 0 && N >= (int64_t)V2D * V2K;
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

// workspace: the split-K partial tiles (S > 1), or the lockstep counters of
// the persistent one-split launch
size_t gram_ws_bytes(int64_t N, int64_t d, int32_t dtype) {
  int T, ntiles, S;
  int64_t nstages;
  plan(N, d, dtype, T, ntiles, S, nstages);
  const int ts = (dtype == KRONQ_BF16) ? BT : FT;
  if (S == 1) return sync_launch(N, d, dtype) ? (size_t)kXcds * kSyncStride * sizeof(unsigned) : 0;
  return (size_t)ntiles * (size_t)S * (size_t)ts * (size_t)ts * sizeof(float);
}

namespace {

// The direct-to-LDS pipeline addresses a lane's load within a stage with an
// unsigned 32-bit byte offset (up to V2K - 1 rows of the operand's pitch)
bool lds_offsets_fit(int64_t lda) { return lda * 2 * V2K + 1024 <= (int64_t(1) << 32); }

// One launch of the split-K scheme for rows [0, p.N) of p.A with the split
// count already planned; `kind` 0 = direct-to-LDS bf16 pipeline (N a multiple
// of V2K, d a multiple of 256), 1 = generic bf16, 2 = fp32.
kronq_status launch_gram(GramParams p, int kind, hipStream_t s) {
  p.nitems = p.ntiles * p.S;
  p.per_xcd = (p.nitems + kXcds - 1) / kXcds;
  const int grid = p.per_xcd * kXcds;
  if (kind == 0 && p.S == 1) {
    unsigned* ctr = static_cast<unsigned*>(static_cast<void*>(p.part));
    hipLaunchKernelGGL(gram_sync_clear, dim3(1), dim3(64), 0, s, ctr);
    KQ_LAUNCHED("gram_sync_clear");
    hipLaunchKernelGGL(gram_bf16_lds_sync_kernel, dim3(kCUs), dim3(BTHREADS), 0, s, p, ctr);
    KQ_LAUNCHED("gram_bf16_lds_sync_kernel");
  } else if (kind == 0) {
    const int ngroups = (p.nitems + 31) / 32;
    const int rgrid = 32 * kXcds * ((ngroups + kXcds - 1) / kXcds);
    hipLaunchKernelGGL(gram_bf16_lds_kernel, dim3(rgrid), dim3(BTHREADS), 0, s, p);
    KQ_LAUNCHED("gram_bf16_lds_kernel");
  } else if (kind == 1) {
    const size_t lds = 4 * PANEL * sizeof(uint16_t);
    if (p.d % 8 == 0) {
      KQ_HIP(hipFuncSetAttribute((const void*)gram_bf16_kernel<false>,
                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
      hipLaunchKernelGGL(gram_bf16_kernel<false>, dim3(grid), dim3(BTHREADS), lds, s, p);
    } else {
      KQ_HIP(hipFuncSetAttribute((const void*)gram_bf16_kernel<true>,
                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
      hipLaunchKernelGGL(gram_bf16_kernel<true>, dim3(grid), dim3(BTHREADS), lds, s, p);
    }
    KQ_LAUNCHED("gram_bf16_kernel");
  } else {
    const size_t lds = 4 * FPANEL * sizeof(float);
    hipLaunchKernelGGL(gram_f32_kernel, dim3(grid), dim3(256), lds, s, p);
    KQ_LAUNCHED("gram_f32_kernel");
  }
  if (p.S > 1) {
    if (kind == 2)
      hipLaunchKernelGGL(gram_finalize_kernel<FT>, dim3(p.ntiles * (FT / 64) * (FT / 64)), dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL(gram_finalize_kernel<BT>, dim3(p.ntiles * (BT / 64) * (BT / 64)), dim3(256), 0, s, p);
    KQ_LAUNCHED("gram_finalize_kernel");
  }
  return KRONQ_OK;
}

}  // namespace

kronq_status gram_launch(const void* A, int32_t dtype, int64_t N, int64_t d, int64_t lda, float* H,
                         int64_t ldh, float scale, float beta, void* ws, size_t ws_bytes,
                         hipStream_t s) {
  (void)ws_bytes;
  GramParams p{};
  p.A = A;
  p.B = A;
  p.N = N;
  p.d = d;
  p.lda = lda;
  p.ldh = ldh;
  p.H = H;
  p.vec_h = ldh % 4 == 0 && reinterpret_cast<uintptr_t>(H) % 16 == 0;
  p.part = static_cast<float*>(ws);
  p.scale = scale;
  p.beta = beta;
  plan(N, d, dtype, p.T, p.ntiles, p.S, p.nstages);
  if (dtype != KRONQ_BF16) return launch_gram(p, 2, s);
  if (d % BT != 0 || !lds_offsets_fit(lda)) return launch_gram(p, 1, s);
  // whole units of V2D stages (128 tokens) through the direct-to-LDS
  // pipeline, then the remaining < 128 tokens accumulated by the generic
  // kernel (beta = 1)
  const int64_t unit = (int64_t)V2D * V2K;
  const int64_t Nmain = N / unit * unit;
  if (Nmain > 0) {
    GramParams q = p;
    q.N = Nmain;
    q.S = (int)std::min<int64_t>(p.S, Nmain / unit);
    kronq_status st = launch_gram(q, 0, s);
    if (st) return st;
  }
  if (N > Nmain) {
    GramParams q = p;
    q.A = static_cast<const uint16_t*>(A) + Nmain * lda;
    q.N = N - Nmain;
    q.S = 1;
    q.nstages = 1;
    if (Nmain > 0) q.beta = 1.0f;
    return launch_gram(q, 1, s);
  }
  return KRONQ_OK;
}

// ------------------------------------------------------------- cross product
//
// C = scale A^T B + beta C - sub for two N x d bf16 matrices with the same
// layout: the same pipelined tiles over all T x T tiles (no symmetry, no
// mirroring).

namespace {

void plan_cross(int64_t N, int64_t d, int& T, int& ntiles, int& S, int64_t& nstages) {
  T = (int)(d / BT);
  ntiles = T * T;
  nstages = N / BK;
  S = choose_splits(ntiles, nstages);
}

}  // namespace

bool gram_pipeline_ld_ok(int64_t ld) { return lds_offsets_fit(ld); }

size_t gram_cross_ws_bytes(int64_t N, int64_t d) {
  int T, ntiles, S;
  int64_t nstages;
  plan_cross(N, d, T, ntiles, S, nstages);
  const int64_t units = N / ((int64_t)V2D * V2K);
  S = (int)std::max<int64_t>(1, std::min<int64_t>(S, units));
  if (S == 1) return (size_t)kXcds * kSyncStride * sizeof(unsigned);
  return (size_t)ntiles * (size_t)S * (size_t)BT * (size_t)BT * sizeof(float);
}

kronq_status gram_cross_launch(const void* A, const void* B, int64_t N, int64_t d, int64_t ld, float* C,
                               int64_t ldc, float scale, float beta, const float* sub, int64_t ldsub,
                               void* ws, hipStream_t s) {
  GramParams p{};
  p.A = A;
  p.B = B;
  p.N = N;
  p.d = d;
  p.lda = ld;
  p.ldh = ldc;
  p.H = C;
  p.sub = sub;
  p.ldsub = ldsub;
  p.cross = true;
  p.vec_h = ldc % 4 == 0 && reinterpret_cast<uintptr_t>(C) % 16 == 0 &&
            (!sub || (ldsub % 4 == 0 && reinterpret_cast<uintptr_t>(sub) % 16 == 0));
  p.part = static_cast<float*>(ws);
  p.scale = scale;
  p.beta = beta;
  if (!lds_offsets_fit(ld))
    return fail(KRONQ_EUNSUPPORTED, "cross product: leading dimension %lld too large for 32-bit "
                "stage offsets (at most %lld)", (long long)ld,
                (long long)(((int64_t(1) << 32) - 1024) / (2 * V2K)));
  plan_cross(N, d, p.T, p.ntiles, p.S, p.nstages);
  p.S = (int)std::max<int64_t>(1, std::min<int64_t>(p.S, N / ((int64_t)V2D * V2K)));
  return launch_gram(p, 0, s);
}

}  // namespace kronq
