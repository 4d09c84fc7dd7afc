// Bidirectional incoherence processing: S_G rescale and randomized block
// Hadamard transforms on both sides of W, H_X and H_G (hyper.ai summary of the
// KronQ paper, Method; Pith review, proof of Theorem 1: W' = U W V^T,
// H_G' = U H_G U^T, H_X' = V H_X V^T).
//
// Every transform here has the form  M <- (I (x) H_kr) Dr M Dc (I (x) H_kc) / sqrt(kr kc)
// for an R x C matrix M: Dr, Dc diagonal (signs, times the S_G rescale where
// it applies), H_k Sylvester Hadamard matrices of order k mixing contiguous
// blocks of rows (kr) and of columns (kc).  The inverse used by the deploy path
// (S_G^-1 U^T W' V) has the factors on the other side,
// M <- Dr (I (x) H_kr) M (I (x) H_kc) Dc / sqrt(kr kc): the same passes with Dc
// applied when pass 1 stores and Dr when the last pass stores.  Because H_kr = H_{kr/R1} (x) H_R1 in
// Sylvester order, the mixing splits into factors that act on separate bits
// of the (row, column) index and commute, so the whole 2-D transform runs in
// two read-modify-write passes over HBM:
//   pass 1: a tile of R1 consecutive rows x C1 columns (C1 = kc, or a few
//           whole column blocks so that a tile row spans at least 64 bytes when
//           kc is small); applies Dr, Dc, the full column-side transform and
//           the low R1 part of the row-side transform (R1 * C1 <= tile size);
//   pass 2: a tile of kr/R1 rows at stride R1 x a strip of CW columns; applies
//           the remaining kr/R1 part of the row-side transform (skipped when
//           R1 == kr).
// Each pass stages its tile (up to 2^14 floats = 64 KiB, so that two
// workgroups share a CU; 2^15 for a pass 2 whose strips would otherwise be
// under 128 bytes) in LDS and runs the butterflies radix-16: a thread gathers
// 16 elements differing in 4 index bits, does 4 butterfly stages in registers
// and scatters them back.  HBM traffic is float4 and coalesced (rows of a
// column block are contiguous; pass-2 strips are whole 16-byte chunks).  LDS rows
// are padded by 4 floats per 32 so that float4-aligned accesses stay 16-byte
// aligned and the low-bit rounds are bank-conflict free.  The forward
// transform of W, H_X and H_G runs as two persistent launches, pass 1 of all
// three and then pass 2 of all three (biip_pass1m / biip_pass2m); the
// inverse, widths that are not a multiple of 4 and large problems (more than
// kMergeMaxTiles pass-1 tiles) run one matrix at a time.
#include "kronq_internal.h"
#include "wht_lds.h"

namespace kronq {
namespace {

constexpr int LOG_TILE = 14;   // 64 KiB tiles: two workgroups per CU overlap HBM and LDS phases
constexpr int TILE = 1 << LOG_TILE;
constexpr int NT = 512;
constexpr int kXcds = 8;

struct Side {
  int64_t block;
  const float* fac;   // per-index factor (signs [* rescale]); never NULL
};

struct TParams {
  float* M;
  int64_t R, C, ld;
  Side row, col;
  int64_t R1;          // low row-block factor handled by pass 1
  int lg_kc, lg_r1;    // log2 of kc and R1
  int lg_c1;           // log2 of the pass-1 tile width C1 (a multiple of kc)
  int lg_rows2;        // log2(kr / R1)
  int lg_cw;           // pass-2 strip width (log2)
  int64_t strips;      // pass-2 strips per row of blocks
  float norm1, norm2;
  bool post;           // factors after the transform (inverse) instead of before
  int64_t tiles1, tiles2;
  int per_xcd1, per_xcd2;
};

__device__ __forceinline__ bool xcd_tile(int64_t ntiles, int per_xcd, int64_t& t) {
  const int b = blockIdx.x;
  t = (int64_t)(b % kXcds) * per_xcd + b / kXcds;
  return (b / kXcds) < per_xcd && t < ntiles;
}

// ---------------------------------------------------------------- vector passes
//
// 256 threads, each holding 16 float4 chunks of the tile: element
//   e = 4 * (t + 256 * i) + j    (j < 4 inside a chunk, thread t < 256, chunk i < 16)
// so index bits 0-1 (j) and 10-13 (i) sit in a thread's registers and bits 2-9
// (t) across threads.  Loads of the whole tile (data and the factors a load
// applies) are issued before anything else, from clamped addresses (chunks past
// the tile read its first element and are dropped).  The butterflies over the
// register bits run in registers, then bits 2-9 in at most two LDS rounds at
// compile-time offsets, then the tile goes back to HBM.  Half the VALU work and
// 40% less LDS traffic than running every bit through LDS.
constexpr int NTB = 256;
constexpr int ECH = TILE / (4 * NTB);   // 16 chunks a thread

__device__ __forceinline__ float4 ld4(const float* a) { return *reinterpret_cast<const float4*>(a); }
__device__ __forceinline__ float4 mul4(float4 a, float4 b, float g) {
  return make_float4(a.x * b.x * g, a.y * b.y * g, a.z * b.z * g, a.w * b.w * g);
}
__device__ __forceinline__ void bfly(float& a, float& b) {
  const float u = a, v = b;
  a = u + v;
  b = u - v;
}

// butterflies over the register bits: lo bit 0 / 1 (inside a chunk) when set in
// mask_lo; chunk bit k (element bit 10 + k) when set in mask_i and 2^k < nch
__device__ __forceinline__ void reg_stages(float4 (&x)[ECH], int nch, int mask_lo, int mask_i) {
  if (mask_lo & 1) {
#pragma unroll
    for (int i = 0; i < ECH; ++i) {
      bfly(x[i].x, x[i].y);
      bfly(x[i].z, x[i].w);
    }
  }
  if (mask_lo & 2) {
#pragma unroll
    for (int i = 0; i < ECH; ++i) {
      bfly(x[i].x, x[i].z);
      bfly(x[i].y, x[i].w);
    }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int h = 1 << k;
    if (h < nch && ((mask_i >> k) & 1)) {
#pragma unroll
      for (int i = 0; i < ECH; ++i)
        if ((i & h) == 0) {
          bfly(x[i].x, x[i + h].x);
          bfly(x[i].y, x[i + h].y);
          bfly(x[i].z, x[i + h].z);
          bfly(x[i].w, x[i + h].w);
        }
    }
  }
}

// one LDS round over bits [b, b + k) of a 2^p tile, b in 2..10 at compile time
template <int NTH = NTB>
__device__ __forceinline__ void lds_round_mid(float* s, int p, int b, int k) {
  switch (b) {
    case 2: lds_round_k<NTH, 2>(s, p, k); break;
    case 3: lds_round_k<NTH, 3>(s, p, k); break;
    case 4: lds_round_k<NTH, 4>(s, p, k); break;
    case 5: lds_round_k<NTH, 5>(s, p, k); break;
    case 6: lds_round_k<NTH, 6>(s, p, k); break;
    case 7: lds_round_k<NTH, 7>(s, p, k); break;
    case 8: lds_round_k<NTH, 8>(s, p, k); break;
    case 9: lds_round_k<NTH, 9>(s, p, k); break;
    default: lds_round_k<NTH, 10>(s, p, k); break;
  }
}

// bits [lo, hi) of the tile through LDS (2 <= lo, hi <= 2 + log2 NTH): the
// thread-index bits, at most two rounds for 256 threads, three for 512
template <int NTH = NTB>
__device__ __forceinline__ void lds_mid_bits(float* s, int p, int lo, int hi) {
  for (int b = lo; b < hi; b += 4) {
    lds_round_mid<NTH>(s, p, b, min(4, hi - b));
    __syncthreads();
  }
}

// whether element bit b of a pass-1 tile is transformed: inside [0, lg), and
// not a column-block index bit (bits [lg_kc, lg_c1) when a tile spans blocks)
__device__ __forceinline__ bool p1_bit(const TParams& p, int lg, int b) {
  return b < lg && (b < p.lg_kc || b >= p.lg_c1);
}

// pass 1: tile = R1 rows x C1 columns, index e = rr * C1 + cc
__global__ void __launch_bounds__(NTB) biip_pass1v(TParams p) {
  extern __shared__ __align__(16) float s[];
  int64_t t;
  if (!xcd_tile(p.tiles1, p.per_xcd1, t)) return;
  const int64_t c1 = int64_t(1) << p.lg_c1;
  const int64_t nb = p.C / c1;
  const int64_t r0 = (t / nb) * p.R1, c0 = (t % nb) * c1;
  const int lg = p.lg_c1 + p.lg_r1;
  const float* cf = p.col.fac;   // NULL: no column factor (identity side)
  const float* rf = p.row.fac;
  const int E = 1 << lg;
  const int nch = E >= 4 * NTB ? E / (4 * NTB) : 1;
  const float4 one4 = make_float4(1.f, 1.f, 1.f, 1.f);
  const float* Mt = p.M + r0 * p.ld + c0;
  int rowi[ECH], coli[ECH];
  float4 x[ECH], f[ECH];
  float g[ECH];
#pragma unroll
  for (int i = 0; i < ECH; ++i) {
    const int e0 = 4 * ((int)threadIdx.x + NTB * i);
    const int e = e0 < E ? e0 : 0;
    rowi[i] = e >> p.lg_c1;
    coli[i] = e & (int)(c1 - 1);
    x[i] = ld4(Mt + (int64_t)rowi[i] * p.ld + coli[i]);
    f[i] = one4;
    g[i] = 1.f;
  }
  if (!p.post) {
    if (cf) {
#pragma unroll
      for (int i = 0; i < ECH; ++i) f[i] = ld4(cf + c0 + coli[i]);
    }
#pragma unroll
    for (int i = 0; i < ECH; ++i) g[i] = rf[r0 + rowi[i]];
  }
#pragma unroll
  for (int i = 0; i < ECH; ++i) x[i] = mul4(x[i], f[i], g[i]);
  int mask_i = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) mask_i |= p1_bit(p, lg, 10 + k) ? (1 << k) : 0;
  reg_stages(x, nch, (p1_bit(p, lg, 0) ? 1 : 0) | (p1_bit(p, lg, 1) ? 2 : 0), mask_i);
#pragma unroll
  for (int i = 0; i < ECH; ++i) {
    const int e0 = 4 * ((int)threadIdx.x + NTB * i);
    if (e0 < E) *reinterpret_cast<float4*>(s + pad(e0)) = x[i];
  }
  __syncthreads();
  // bits 2-9: the column bits below kc, and the bits from C1 up
  const int hi = min(lg, 10);
  if (p.lg_c1 == p.lg_kc) {
    lds_mid_bits(s, lg, 2, hi);
  } else {
    lds_mid_bits(s, lg, 2, min(p.lg_kc, hi));
    lds_mid_bits(s, lg, max(p.lg_c1, 2), hi);
  }
  const float nrm = p.norm1;
  // inverse: Dc always lands here (the column transform is complete); Dr only
  // when no second pass follows
  const bool post_c = p.post && cf, post_r = p.post && p.tiles2 == 0;
#pragma unroll
  for (int i = 0; i < ECH; ++i) {
    f[i] = one4;
    g[i] = nrm;
  }
  if (post_c) {
#pragma unroll
    for (int i = 0; i < ECH; ++i) f[i] = ld4(cf + c0 + coli[i]);
  }
  if (post_r) {
#pragma unroll
    for (int i = 0; i < ECH; ++i) g[i] = nrm * rf[r0 + rowi[i]];
  }
#pragma unroll
  for (int i = 0; i < ECH; ++i) {
    const int e0 = 4 * ((int)threadIdx.x + NTB * i);
    if (e0 < E) {
      const float4 y = *reinterpret_cast<const float4*>(s + pad(e0));
      *reinterpret_cast<float4*>(p.M + (r0 + rowi[i]) * p.ld + c0 + coli[i]) = mul4(y, f[i], g[i]);
    }
  }
}

// pass 2: tile = (kr / R1) rows at stride R1 x CW columns, index e = j * CW + c;
// the transformed bits are the row bits [lg_cw, lg).  NTH threads of 16 float4
// chunks: tiles of up to 2^14 elements with 256 threads, 2^15 with 512 (the
// wide form: twice the strip width, 144 KiB of LDS, one workgroup per CU).
// Element e = 4 * (t + NTH * i) + j, so chunk bit k is element bit CB + k.
template <int NTH>
__global__ void __launch_bounds__(NTH) biip_pass2v(TParams p) {
  constexpr int CB = NTH == 512 ? 11 : 10;
  static_assert(NTH == 256 || NTH == 512, "pass 2 runs 256 or 512 threads");
  extern __shared__ __align__(16) float s[];
  int64_t t;
  if (!xcd_tile(p.tiles2, p.per_xcd2, t)) return;
  const int64_t kr = p.row.block;
  const int64_t strip = t % p.strips;
  const int64_t rest = t / p.strips;
  const int64_t res = rest % p.R1, rb = rest / p.R1;
  const int64_t rbase = rb * kr + res;
  const int64_t cbase = strip << p.lg_cw;
  const int lg = p.lg_rows2 + p.lg_cw;
  const int E = 1 << lg;
  const int nch = E >= 4 * NTH ? E / (4 * NTH) : 1;
  const int64_t cmask = (1 << p.lg_cw) - 1;
  float4 x[ECH];
#pragma unroll
  for (int i = 0; i < ECH; ++i) {
    const int e0 = 4 * ((int)threadIdx.x + NTH * i);
    const int64_t j = e0 >> p.lg_cw, c = cbase + (e0 & cmask);
    const bool in = e0 < E && c < p.C;
    const float4 v = ld4(p.M + (in ? (rbase + j * p.R1) * p.ld + c : rbase * p.ld + cbase));
    x[i] = in ? v : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  int mask_i = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) mask_i |= (CB + k >= p.lg_cw && CB + k < lg) ? (1 << k) : 0;
  reg_stages(x, nch, 0, mask_i);   // bits 0-1 are column bits (cw >= 4)
#pragma unroll
  for (int i = 0; i < ECH; ++i) {
    const int e0 = 4 * ((int)threadIdx.x + NTH * i);
    if (e0 < E) *reinterpret_cast<float4*>(s + pad(e0)) = x[i];
  }
  __syncthreads();
  lds_mid_bits<NTH>(s, lg, max(p.lg_cw, 2), min(lg, CB));
  const float nrm = p.norm2;
  float g[ECH];
#pragma unroll
  for (int i = 0; i < ECH; ++i) g[i] = nrm;
  if (p.post) {
#pragma unroll
    for (int i = 0; i < ECH; ++i) {
      const int e0 = 4 * ((int)threadIdx.x + NTH * i);
      const int64_t j = e0 < E ? (e0 >> p.lg_cw) : 0;
      g[i] = nrm * p.row.fac[rbase + j * p.R1];
    }
  }
#pragma unroll
  for (int i = 0; i < ECH; ++i) {
    const int e0 = 4 * ((int)threadIdx.x + NTH * i);
    const int64_t j = e0 >> p.lg_cw, c = cbase + (e0 & cmask);
    if (e0 < E && c < p.C) {
      const float4 y = *reinterpret_cast<const float4*>(s + pad(e0));
      const float f = g[i];
      *reinterpret_cast<float4*>(p.M + (rbase + j * p.R1) * p.ld + c) =
          make_float4(y.x * f, y.y * f, y.z * f, y.w * f);
    }
  }
}

// ---------------------------------------------------------------- merged forward passes
//
// The forward transform of up to three matrices (W, H_X, H_G) in two launches:
// pass 1 of every matrix, then pass 2 of every matrix.  The grid is persistent,
// two workgroups per CU, each walking a run of tiles.  A workgroup issues the
// next tile's loads (into the registers the current tile has just left) as
// soon as the current tile sits in LDS, so its HBM reads overlap the LDS
// butterflies and the stores of the tile before; one tile per workgroup and
// launch would instead run every workgroup's load, butterfly and store phases
// in lockstep and leave HBM idle during the butterflies.  Tiles are numbered
// matrix after matrix and XCD x walks the x-th eighth of that list, so
// neighbouring pass-2 strips, which share 128-byte lines, meet in one L2.
// Tiles and butterflies are those of biip_pass1v / biip_pass2v.
constexpr int kSlots = 512;   // 2 workgroups on each of the 256 CUs

struct MultiParams {
  TParams p[3];
  int64_t end1[3], end2[3];   // cumulative pass-1 / pass-2 tile counts
};

__device__ __forceinline__ int owner(const int64_t (&end)[3], int64_t g) {
  return (g >= end[0] ? 1 : 0) + (g >= end[1] ? 1 : 0);
}

// the tiles [lo, hi) of this workgroup's XCD; the workgroup takes every
// nslot-th of them from lo + slot
__device__ __forceinline__ void xcd_run(int64_t total, int64_t& lo, int64_t& hi, int& nslot) {
  const int xcd = blockIdx.x % kXcds;
  nslot = gridDim.x / kXcds;
  const int64_t per = (total + kXcds - 1) / kXcds;
  lo = xcd * per;
  hi = min(total, lo + per);
  lo += blockIdx.x / kXcds;
}

__device__ __forceinline__ void p1_origin(const TParams& p, int64_t t, int64_t& r0, int64_t& c0) {
  const int64_t nb = p.C >> p.lg_c1;
  r0 = (t / nb) * p.R1;
  c0 = (t % nb) << p.lg_c1;
}

// issue the loads of pass-1 tile t: data, column factors (ones when absent),
// row factors.  FULL: every tile holds 2^14 elements (no clamping).
template <bool FULL>
__device__ __forceinline__ void p1_issue(const TParams& p, int64_t t, float4 (&x)[ECH],
                                         float4 (&f)[ECH], float (&g)[ECH]) {
  int64_t r0, c0;
  p1_origin(p, t, r0, c0);
  const int E = FULL ? TILE : 1 << (p.lg_c1 + p.lg_r1);
  const int cm = (1 << p.lg_c1) - 1;
  const float* Mt = p.M + r0 * p.ld + c0;
  const float* cf = p.col.fac;
  const float* rf = p.row.fac + r0;
#pragma unroll
  for (int i = 0; i < ECH; ++i) {
    const int e0 = 4 * ((int)threadIdx.x + NTB * i);
    const int e = e0 < E ? e0 : 0;
    x[i] = ld4(Mt + (int64_t)(e >> p.lg_c1) * p.ld + (e & cm));
  }
  if (cf) {
#pragma unroll
    for (int i = 0; i < ECH; ++i) {
      const int e0 = 4 * ((int)threadIdx.x + NTB * i);
      f[i] = ld4(cf + c0 + ((e0 < E ? e0 : 0) & cm));
    }
  } else {
#pragma unroll
    for (int i = 0; i < ECH; ++i) f[i] = make_float4(1.f, 1.f, 1.f, 1.f);
  }
#pragma unroll
  for (int i = 0; i < ECH; ++i) {
    const int e0 = 4 * ((int)threadIdx.x + NTB * i);
    g[i] = rf[(e0 < E ? e0 : 0) >> p.lg_c1];
  }
}

__device__ __forceinline__ const TParams& tile_of(const MultiParams& mp, const int64_t (&end)[3],
                                                  int64_t g, int64_t& t) {
  const int k = owner(end, g);
  t = g - (k ? end[k - 1] : 0);
  return mp.p[k];
}

// pass-1 tile, loaded: factors, register butterflies, into LDS
template <bool FULL>
__device__ __forceinline__ void p1_stage_in(const TParams& p, float* s, float4 (&x)[ECH],
                                            const float4 (&f)[ECH], const float (&g)[ECH]) {
  const int lg = FULL ? LOG_TILE : p.lg_c1 + p.lg_r1;
  const int E = 1 << lg;
  const int nch = E >= 4 * NTB ? E / (4 * NTB) : 1;
#pragma unroll
  for (int i = 0; i < ECH; ++i) x[i] = mul4(x[i], f[i], g[i]);
  int mask_i = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) mask_i |= p1_bit(p, lg, 10 + b) ? (1 << b) : 0;
  reg_stages(x, nch, (p1_bit(p, lg, 0) ? 1 : 0) | (p1_bit(p, lg, 1) ? 2 : 0), mask_i);
#pragma unroll
  for (int i = 0; i < ECH; ++i) {
    const int e0 = 4 * ((int)threadIdx.x + NTB * i);
    if (e0 < E) *reinterpret_cast<float4*>(s + pad(e0)) = x[i];
  }
  __syncthreads();
}

// pass-1 tile in LDS: the LDS butterflies, then back to HBM.  The stores of a
// FULL tile are unconditional, which lets the next tile's waits leave them in
// flight (a guarded store may not have been issued, so a wait for a load
// issued before it would have to assume it was not).
template <bool FULL>
__device__ __forceinline__ void p1_finish(const TParams& p, int64_t t, float* s) {
  int64_t r0, c0;
  p1_origin(p, t, r0, c0);
  const int lg = FULL ? LOG_TILE : p.lg_c1 + p.lg_r1;
  const int E = 1 << lg;
  const int bhi = min(lg, 10);
  if (p.lg_c1 == p.lg_kc) {
    lds_mid_bits(s, lg, 2, bhi);
  } else {
    lds_mid_bits(s, lg, 2, min(p.lg_kc, bhi));
    lds_mid_bits(s, lg, max(p.lg_c1, 2), bhi);
  }
  const float nrm = p.norm1;
  const int cm = (1 << p.lg_c1) - 1;
  float* Mt = p.M + r0 * p.ld + c0;
#pragma unroll
  for (int i = 0; i < ECH; ++i) {
    const int e0 = 4 * ((int)threadIdx.x + NTB * i);
    if (e0 < E) {
      const float4 y = *reinterpret_cast<const float4*>(s + pad(e0));
      *reinterpret_cast<float4*>(Mt + (int64_t)(e0 >> p.lg_c1) * p.ld + (e0 & cm)) =
          make_float4(y.x * nrm, y.y * nrm, y.z * nrm, y.w * nrm);
    }
  }
}

// The loop is rotated so that inside it the next tile's loads are always
// followed by this tile's stores: the waits for those loads then leave the
// stores in flight.
template <bool FULL>
__global__ void __launch_bounds__(NTB) __attribute__((amdgpu_waves_per_eu(2))) biip_pass1m(MultiParams mp) {
  extern __shared__ __align__(16) float s[];
  int64_t gt, hi, t;
  int nslot;
  xcd_run(mp.end1[2], gt, hi, nslot);
  if (gt >= hi) return;
  float4 x[ECH], f[ECH];
  float g[ECH];
  {
    const TParams& p = tile_of(mp, mp.end1, gt, t);
    p1_issue<FULL>(p, t, x, f, g);
    p1_stage_in<FULL>(p, s, x, f, g);
  }
  for (;;) {
    const TParams& p = tile_of(mp, mp.end1, gt, t);
    const int64_t gn = gt + nslot;
    if (gn >= hi) {
      p1_finish<FULL>(p, t, s);
      break;
    }
    int64_t tn;
    const TParams& pn = tile_of(mp, mp.end1, gn, tn);
    p1_issue<FULL>(pn, tn, x, f, g);
    p1_finish<FULL>(p, t, s);
    __syncthreads();   // every thread has read the tile before the next one is written
    p1_stage_in<FULL>(pn, s, x, f, g);
    gt = gn;
  }
}

struct P2Origin {
  int64_t rbase, cbase;
};

__device__ __forceinline__ P2Origin p2_origin(const TParams& p, int64_t t) {
  const int64_t strip = t % p.strips;
  const int64_t rest = t / p.strips;
  return P2Origin{(rest / p.R1) * p.row.block + rest % p.R1, strip << p.lg_cw};
}

// issue the loads of pass-2 tile t.  Columns past C read a valid element of
// the tile instead; pass 2 mixes only the row bits, so such a column never
// meets a valid one and is never stored.  FULL: every tile holds 2^14
// elements and every strip lies inside the matrix.
template <bool FULL>
__device__ __forceinline__ void p2_issue(const TParams& p, int64_t t, float4 (&x)[ECH]) {
  const P2Origin o = p2_origin(p, t);
  const int E = FULL ? TILE : 1 << (p.lg_rows2 + p.lg_cw);
  const int cm = (1 << p.lg_cw) - 1;
  const float* base = p.M + o.rbase * p.ld + o.cbase;
  const int64_t rstride = p.R1 * p.ld;
#pragma unroll
  for (int i = 0; i < ECH; ++i) {
    const int e0 = 4 * ((int)threadIdx.x + NTB * i);
    const int e = e0 < E ? e0 : 0;
    const int c = e & cm;
    const bool in = FULL || o.cbase + c < p.C;
    x[i] = ld4(base + (in ? (int64_t)(e >> p.lg_cw) * rstride + c : 0));
  }
}

template <bool FULL>
__device__ __forceinline__ void p2_stage_in(const TParams& p, float* s, float4 (&x)[ECH]) {
  const int lg = FULL ? LOG_TILE : p.lg_rows2 + p.lg_cw;
  const int E = 1 << lg;
  const int nch = E >= 4 * NTB ? E / (4 * NTB) : 1;
  int mask_i = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) mask_i |= (10 + b >= p.lg_cw && 10 + b < lg) ? (1 << b) : 0;
  reg_stages(x, nch, 0, mask_i);   // bits 0-1 are column bits (cw >= 4)
#pragma unroll
  for (int i = 0; i < ECH; ++i) {
    const int e0 = 4 * ((int)threadIdx.x + NTB * i);
    if (e0 < E) *reinterpret_cast<float4*>(s + pad(e0)) = x[i];
  }
  __syncthreads();
}

template <bool FULL>
__device__ __forceinline__ void p2_finish(const TParams& p, int64_t t, float* s) {
  const P2Origin o = p2_origin(p, t);
  const int lg = FULL ? LOG_TILE : p.lg_rows2 + p.lg_cw;
  const int E = 1 << lg;
  lds_mid_bits(s, lg, max(p.lg_cw, 2), min(lg, 10));
  const float nrm = p.norm2;
  const int cm = (1 << p.lg_cw) - 1;
  float* base = p.M + o.rbase * p.ld + o.cbase;
  const int64_t rstride = p.R1 * p.ld;
#pragma unroll
  for (int i = 0; i < ECH; ++i) {
    const int e0 = 4 * ((int)threadIdx.x + NTB * i);
    const int c = e0 & cm;
    if (FULL || (e0 < E && o.cbase + c < p.C)) {
      const float4 y = *reinterpret_cast<const float4*>(s + pad(e0));
      *reinterpret_cast<float4*>(base + (int64_t)(e0 >> p.lg_cw) * rstride + c) =
          make_float4(y.x * nrm, y.y * nrm, y.z * nrm, y.w * nrm);
    }
  }
}

template <bool FULL>
__global__ void __launch_bounds__(NTB) __attribute__((amdgpu_waves_per_eu(2))) biip_pass2m(MultiParams mp) {
  extern __shared__ __align__(16) float s[];
  int64_t gt, hi, t;
  int nslot;
  xcd_run(mp.end2[2], gt, hi, nslot);
  if (gt >= hi) return;
  float4 x[ECH];
  {
    const TParams& p = tile_of(mp, mp.end2, gt, t);
    p2_issue<FULL>(p, t, x);
    p2_stage_in<FULL>(p, s, x);
  }
  for (;;) {
    const TParams& p = tile_of(mp, mp.end2, gt, t);
    const int64_t gn = gt + nslot;
    if (gn >= hi) {
      p2_finish<FULL>(p, t, s);
      break;
    }
    int64_t tn;
    const TParams& pn = tile_of(mp, mp.end2, gn, tn);
    p2_issue<FULL>(pn, tn, x);
    p2_finish<FULL>(p, t, s);
    __syncthreads();   // every thread has read the tile before the next one is written
    p2_stage_in<FULL>(pn, s, x);
    gt = gn;
  }
}

// ---------------------------------------------------------------- scalar passes
// (widths that are not a multiple of 4): one element a thread at a time

// pass 1: tile = R1 rows x C1 columns, index e = rr * C1 + cc
__global__ void __launch_bounds__(NT) biip_pass1s(TParams p) {
  extern __shared__ __align__(16) float s[];
  int64_t t;
  if (!xcd_tile(p.tiles1, p.per_xcd1, t)) return;
  const int64_t c1 = int64_t(1) << p.lg_c1;
  const int64_t nb = p.C / c1;
  const int64_t r0 = (t / nb) * p.R1, c0 = (t % nb) * c1;
  const int lg = p.lg_c1 + p.lg_r1;
  const float* cf = p.col.fac;
  const float* rf = p.row.fac;
  const int E = 1 << lg;
  for (int e = threadIdx.x; e < E; e += NT) {
    const int64_t rr = e >> p.lg_c1, cc = e & (c1 - 1);
    const int64_t r = r0 + rr, c = c0 + cc;
    const float x = p.M[r * p.ld + c];
    s[pad(e)] = p.post ? x : x * (cf ? cf[c] : 1.f) * rf[r];
  }
  __syncthreads();
  if (p.lg_c1 == p.lg_kc) {
    lds_wht_bits<NT>(s, lg, 0, lg);
  } else {
    lds_wht_bits<NT>(s, lg, 0, p.lg_kc);
    lds_wht_bits<NT>(s, lg, p.lg_c1, lg);
  }
  const float nrm = p.norm1;
  const bool post_c = p.post && cf, post_r = p.post && p.tiles2 == 0;
  for (int e = threadIdx.x; e < E; e += NT) {
    const int64_t rr = e >> p.lg_c1, cc = e & (c1 - 1);
    float f = nrm;
    if (post_c) f *= cf[c0 + cc];
    if (post_r) f *= rf[r0 + rr];
    p.M[(r0 + rr) * p.ld + c0 + cc] = s[pad(e)] * f;
  }
}

// pass 2: tile = (kr / R1) rows at stride R1 x CW columns, index e = j * CW + c
__global__ void __launch_bounds__(NT) biip_pass2s(TParams p) {
  extern __shared__ __align__(16) float s[];
  int64_t t;
  if (!xcd_tile(p.tiles2, p.per_xcd2, t)) return;
  const int64_t kr = p.row.block;
  const int64_t strip = t % p.strips;
  const int64_t rest = t / p.strips;
  const int64_t res = rest % p.R1, rb = rest / p.R1;
  const int64_t rbase = rb * kr + res;
  const int64_t cbase = strip << p.lg_cw;
  const int lg = p.lg_rows2 + p.lg_cw;
  const int E = 1 << lg;
  const int64_t cmask = (1 << p.lg_cw) - 1;
  for (int e = threadIdx.x; e < E; e += NT) {
    const int64_t j = e >> p.lg_cw, c = cbase + (e & cmask);
    s[pad(e)] = (c < p.C) ? p.M[(rbase + j * p.R1) * p.ld + c] : 0.f;
  }
  __syncthreads();
  lds_wht_bits<NT>(s, lg, p.lg_cw, lg);
  const float nrm = p.norm2;
  for (int e = threadIdx.x; e < E; e += NT) {
    const int64_t j = e >> p.lg_cw, c = cbase + (e & cmask);
    if (c < p.C) {
      const int64_t r = rbase + j * p.R1;
      p.M[r * p.ld + c] = s[pad(e)] * (p.post ? nrm * p.row.fac[r] : nrm);
    }
  }
}

// sg[i] = HG[i][i]^alpha (1 when not positive or alpha == 0);
// rfW[i] = so[i] * sg[i];  rfG[i] = so[i] / sg[i]
__global__ void biip_prep(const float* HG, int64_t ldhg, int64_t m, float alpha, const float* so,
                          float* sg_ws, float* rfW, float* rfG, float* sg_out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= m) return;
  float g = 1.0f;
  if (alpha != 0.0f) {
    const float dgi = HG[i * ldhg + i];
    if (dgi > 0.0f) g = powf(dgi, alpha);
  }
  sg_ws[i] = g;
  const float o = so ? so[i] : 1.f;   // NULL: identity output side
  rfW[i] = o * g;
  rfG[i] = o / g;
  if (sg_out) sg_out[i] = g;
}

// input-side rescale: sx[j] = sx_in[j] when given, else HX[j][j]^alpha_x
// (1 when not positive or alpha_x == 0), read before any transform;
// cfW[j] = si[j] * sx[j] (W's columns), cfX[j] = si[j] / sx[j] (both sides of H_X)
__global__ void biip_prep_in(const float* HX, int64_t ldhx, int64_t n, float alpha_x,
                             const float* sx_in, const float* si, float* cfW, float* cfX,
                             float* sx_out) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n) return;
  float x = 1.0f;
  if (sx_in) {
    x = sx_in[j];
  } else if (alpha_x != 0.0f) {
    const float dxj = HX[j * ldhx + j];
    if (dxj > 0.0f) x = powf(dxj, alpha_x);
  }
  const float o = si ? si[j] : 1.f;   // NULL: identity input side
  cfW[j] = o * x;
  cfX[j] = o / x;
  if (sx_out && !sx_in) sx_out[j] = x;
}

// cf[j] = si[j] / sx[j]: the column factor of the inverse with an input rescale
__global__ void unrotate_prep_in(const float* si, const float* sx, int64_t n, float* cf) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n) return;
  cf[j] = (si ? si[j] : 1.f) / sx[j];
}

// rf[i] = so[i] / sg[i]  (sg NULL: all ones)
__global__ void unrotate_prep(const float* so, const float* sg, int64_t m, float* rf) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= m) return;
  const float o = so ? so[i] : 1.f;   // NULL: identity output side
  rf[i] = sg ? o / sg[i] : o;
}

int ilog2(int64_t x) {
  int l = 0;
  while ((int64_t(1) << l) < x) ++l;
  return l;
}

int64_t pow2_floor(int64_t x) {
  int64_t p = 1;
  while (p * 2 <= x) p *= 2;
  return p;
}

struct Plan {
  TParams p;
  bool vec1, vec2;
};

Plan plan2d(float* M, int64_t R, int64_t C, int64_t ld, int64_t kr, const float* rfac, int64_t kc,
            const float* cfac, bool post) {
  Plan pl{};
  TParams& p = pl.p;
  p.post = post;
  p.M = M;
  p.R = R;
  p.C = C;
  p.ld = ld;
  p.row = Side{kr, rfac};
  p.col = Side{kc, cfac};
  // pass-1 tile width: whole column blocks, at least 16 columns (64 bytes)
  // where the width allows, so that a block of 1 does not read single columns
  int64_t c1 = kc;
  while (c1 < 16 && (C / kc) % (2 * c1 / kc) == 0) c1 *= 2;
  p.lg_c1 = ilog2(c1);
  p.R1 = std::min<int64_t>(kr, TILE / c1);
  p.lg_kc = ilog2(kc);
  p.lg_r1 = ilog2(p.R1);
  const int64_t rows2 = kr / p.R1;
  p.lg_rows2 = ilog2(rows2);
  p.norm1 = (float)(1.0 / std::sqrt((double)(p.R1 * kc)));
  p.norm2 = (float)(1.0 / std::sqrt((double)rows2));
  const int64_t cw = std::min<int64_t>(pow2_floor(C), TILE / rows2);
  p.lg_cw = ilog2(cw);
  p.strips = (C + cw - 1) / cw;
  p.tiles1 = (R / p.R1) * (C / c1);
  p.tiles2 = (rows2 > 1) ? (R / kr) * p.R1 * p.strips : 0;
  p.per_xcd1 = (int)((p.tiles1 + kXcds - 1) / kXcds);
  p.per_xcd2 = (int)((p.tiles2 + kXcds - 1) / kXcds);
  pl.vec1 = (c1 % 4 == 0) && (ld % 4 == 0) && ((uintptr_t)M % 16 == 0) &&
            ((uintptr_t)cfac % 16 == 0);
  pl.vec2 = (cw % 4 == 0) && (C % 4 == 0) && (ld % 4 == 0) && ((uintptr_t)M % 16 == 0);
  return pl;
}

// Pass-2 strips narrower than 128 bytes (cw < 32) are doubled where the
// matrix is wide enough, with tiles of 2^15 elements (the 512-thread pass 2).
// Measured on a 28672^2 matrix (column block 4096, pass 1 unchanged), pass 2
// took 1.46-1.50 ms with 64-byte strips, 1.31 ms with 128-byte and 1.28 ms
// with 256-byte strips.
bool widen_pass2(TParams& p) {
  const int64_t cw = int64_t(1) << p.lg_cw;
  if (cw >= 32 || pow2_floor(p.C) < 2 * cw || p.lg_rows2 + p.lg_cw != LOG_TILE) return false;
  p.lg_cw += 1;
  p.strips = (p.C + 2 * cw - 1) / (2 * cw);
  p.tiles2 = (p.R / p.row.block) * p.R1 * p.strips;
  p.per_xcd2 = (int)((p.tiles2 + kXcds - 1) / kXcds);
  return true;
}

// one matrix, one workgroup per tile
kronq_status launch2d(const Plan& pl, hipStream_t st) {
  TParams p = pl.p;
  const size_t lds1 = padded(1 << (p.lg_c1 + p.lg_r1)) * sizeof(float);
  const size_t ldsmax = padded(TILE) * sizeof(float);
  {
    auto k1 = pl.vec1 ? biip_pass1v : biip_pass1s;
    KQ_HIP(hipFuncSetAttribute((const void*)k1, hipFuncAttributeMaxDynamicSharedMemorySize, (int)ldsmax));
    hipLaunchKernelGGL(k1, dim3(p.per_xcd1 * kXcds), dim3(pl.vec1 ? NTB : NT), lds1, st, p);
    KQ_LAUNCHED("biip_pass1");
  }
  if (p.tiles2) {
    const bool wide = pl.vec2 && widen_pass2(p);
    const size_t lds2 = padded(1 << (p.lg_rows2 + p.lg_cw)) * sizeof(float);
    auto k2 = wide ? biip_pass2v<512> : pl.vec2 ? biip_pass2v<NTB> : biip_pass2s;
    const size_t lmax = wide ? padded(2 * TILE) * sizeof(float) : ldsmax;
    KQ_HIP(hipFuncSetAttribute((const void*)k2, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lmax));
    hipLaunchKernelGGL(k2, dim3(p.per_xcd2 * kXcds), dim3(wide ? 512 : pl.vec2 ? NTB : NT), lds2, st, p);
    KQ_LAUNCHED("biip_pass2");
  }
  return KRONQ_OK;
}

// forward transforms of n <= 3 matrices: the merged persistent passes when
// every matrix takes the vector path, else one matrix at a time
// Up to this many pass-1 tiles in all, the merged persistent passes are
// faster; above it a launch per matrix and pass is (measured, W + H_X + H_G:
// 4096^2 0.162 ms merged against 0.200 per matrix, 1024 x 4096 0.085 against
// 0.121; 4096 x 11008 (11172 tiles) 0.723 against 0.617, 14336 x 4096 1.034
// against 0.895, 28672 x 8192 and 8192 x 28672 6.12 against 4.01-4.07).
constexpr int64_t kMergeMaxTiles = 4096;

kronq_status launch_forward(const Plan* pl, int n, hipStream_t st) {
  bool merged = n > 0;
  int64_t all1 = 0;
  for (int k = 0; k < n; ++k) {
    merged = merged && !pl[k].p.post && pl[k].p.row.fac && pl[k].vec1 &&
             (pl[k].vec2 || pl[k].p.tiles2 == 0);
    all1 += pl[k].p.tiles1;
  }
  merged = merged && all1 <= kMergeMaxTiles;
  if (!merged) {
    for (int k = 0; k < n; ++k) {
      const kronq_status s = launch2d(pl[k], st);
      if (s) return s;
    }
    return KRONQ_OK;
  }
  MultiParams mp{};
  int64_t t1 = 0, t2 = 0;
  for (int k = 0; k < 3; ++k) {
    if (k < n) {
      mp.p[k] = pl[k].p;
      t1 += pl[k].p.tiles1;
      t2 += pl[k].p.tiles2;
    }
    mp.end1[k] = t1;
    mp.end2[k] = t2;
  }
  if (t1 == 0) return KRONQ_OK;
  // full tiles everywhere (2^14 elements, pass-2 strips inside the matrix):
  // the variant without bounds checks
  bool full1 = true, full2 = true;
  for (int k = 0; k < n; ++k) {
    const TParams& p = pl[k].p;
    full1 = full1 && p.lg_c1 + p.lg_r1 == LOG_TILE;
    if (p.tiles2)
      full2 = full2 && p.lg_rows2 + p.lg_cw == LOG_TILE && p.C % (int64_t(1) << p.lg_cw) == 0;
  }
  const size_t ldsmax = padded(TILE) * sizeof(float);
  auto grid = [](int64_t tiles) {
    const int64_t g = std::min<int64_t>((tiles + kXcds - 1) / kXcds * kXcds, kSlots);
    return dim3((unsigned)g);
  };
  {
    auto k1 = full1 ? biip_pass1m<true> : biip_pass1m<false>;
    KQ_HIP(hipFuncSetAttribute((const void*)k1, hipFuncAttributeMaxDynamicSharedMemorySize, (int)ldsmax));
    hipLaunchKernelGGL(k1, grid(t1), dim3(NTB), ldsmax, st, mp);
    KQ_LAUNCHED("biip_pass1m");
  }
  if (t2) {
    auto k2 = full2 ? biip_pass2m<true> : biip_pass2m<false>;
    KQ_HIP(hipFuncSetAttribute((const void*)k2, hipFuncAttributeMaxDynamicSharedMemorySize, (int)ldsmax));
    hipLaunchKernelGGL(k2, grid(t2), dim3(NTB), ldsmax, st, mp);
    KQ_LAUNCHED("biip_pass2m");
  }
  return KRONQ_OK;
}

}  // namespace

size_t biip_ws_bytes(int64_t m, int64_t n) {
  (void)n;
  return 3 * align_up((size_t)m * sizeof(float), 256);
}

size_t biip_sx_ws_bytes(int64_t m, int64_t n) {
  return biip_ws_bytes(m, n) + 2 * align_up((size_t)n * sizeof(float), 256);
}

kronq_status biip_launch(float* W, int64_t m, int64_t n, int64_t ldw, float* HX, int64_t ldhx,
                         float* HG, int64_t ldhg, const kronq_had& in, const kronq_had& out,
                         float alpha, float* sg, void* ws, size_t ws_bytes, hipStream_t s,
                         bool rescale_in, float alpha_x, const float* sx_in, float* sx_out) {
  (void)ws_bytes;
  const size_t seg = align_up((size_t)m * sizeof(float), 256);
  float* sg_ws = static_cast<float*>(ws);
  float* rfW = reinterpret_cast<float*>(static_cast<char*>(ws) + seg);
  float* rfG = reinterpret_cast<float*>(static_cast<char*>(ws) + 2 * seg);
  hipLaunchKernelGGL(biip_prep, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, s,
                     (const float*)HG, ldhg, m, alpha, out.signs, sg_ws, rfW, rfG, sg);
  KQ_LAUNCHED("biip_prep");
  // an identity side (block 1, no signs) leaves its factor alone: V = I keeps
  // H_X, U = I without a rescale keeps H_G (and W when both sides are so)
  const bool v_id = in.block == 1 && !in.signs, u_id = out.block == 1 && !out.signs;
  // input rescale: W's columns take si * sx, H_X's rows and columns si / sx
  const float* cfW = in.signs;
  const float* cfX = in.signs;
  if (rescale_in) {
    float* cw = reinterpret_cast<float*>(static_cast<char*>(ws) + 3 * seg);
    float* cx = cw + align_up((size_t)n * sizeof(float), 256) / sizeof(float);
    hipLaunchKernelGGL(biip_prep_in, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       (const float*)HX, ldhx, n, alpha_x, sx_in, in.signs, cw, cx, sx_out);
    KQ_LAUNCHED("biip_prep_in");
    cfW = cw;
    cfX = cx;
  }
  Plan pl[3];
  int n_mat = 0;
  if (W && !(v_id && u_id && alpha == 0.0f && !rescale_in))
    pl[n_mat++] = plan2d(W, m, n, ldw, out.block, rfW, in.block, cfW, false);
  if (HX && !(v_id && !rescale_in))
    pl[n_mat++] = plan2d(HX, n, n, ldhx, in.block, cfX, in.block, cfX, false);
  if (HG && !(u_id && alpha == 0.0f))
    pl[n_mat++] = plan2d(HG, m, m, ldhg, out.block, rfG, out.block, rfG, false);
  return launch_forward(pl, n_mat, s);
}

size_t unrotate_ws_bytes(int64_t m) { return align_up((size_t)m * sizeof(float), 256); }

kronq_status unrotate_launch(float* W, int64_t m, int64_t n, int64_t ldw, const kronq_had& in,
                             const kronq_had& out, const float* sg, void* ws, hipStream_t s) {
  float* rf = static_cast<float*>(ws);
  hipLaunchKernelGGL(unrotate_prep, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, s, out.signs,
                     sg, m, rf);
  KQ_LAUNCHED("unrotate_prep");
  return launch2d(plan2d(W, m, n, ldw, out.block, rf, in.block, in.signs, true), s);
}

size_t unrotate_sx_ws_bytes(int64_t m, int64_t n) {
  return unrotate_ws_bytes(m) + align_up((size_t)n * sizeof(float), 256);
}

kronq_status unrotate_sx_launch(float* W, int64_t m, int64_t n, int64_t ldw, const kronq_had& in,
                                const kronq_had& out, const float* sg, const float* sx, void* ws,
                                hipStream_t s) {
  float* rf = static_cast<float*>(ws);
  float* cf = reinterpret_cast<float*>(static_cast<char*>(ws) + unrotate_ws_bytes(m));
  hipLaunchKernelGGL(unrotate_prep, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, s, out.signs,
                     sg, m, rf);
  KQ_LAUNCHED("unrotate_prep");
  hipLaunchKernelGGL(unrotate_prep_in, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, in.signs,
                     sx, n, cf);
  KQ_LAUNCHED("unrotate_prep_in");
  return launch2d(plan2d(W, m, n, ldw, out.block, rf, in.block, cf, true), s);
}

}  // namespace kronq
