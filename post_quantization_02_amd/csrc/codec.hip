// Deploy codec: packed low-bit codes and the batch-1 decode matvec of a layer
// quantized after bidirectional incoherence processing (GitHub README of the
// KronQ release: int4 / int2 weights stored packed, unpacked on the fly by a
// fused dequantize + BiIP matvec for single-token decode; Pith review,
// Theorem 1: W' = U W V^T; hyper.ai summary, Method: the S_G rescale precedes
// the transforms, so the original-domain weight is S_G^-1 U^T W' V).
//
// Storage of bits 2 and 4: code j of a row sits at bit offset
// bits * (j mod (8 / bits)) of byte j / (8 / bits); a row is padded to whole
// bytes.  Other widths keep one code per byte, as the column loop emits them.
//
// Decode of y = S_G^-1 U^T W^ V x with W^[r][c] = s[r][g] (q[r][c] - z[r][g]),
// two launches:
//   decode_gemv  x' = V x = (I (x) H_kin) D_in x / sqrt(kin) for the
//                workgroup's column slice (LDS butterflies), then
//                P[t][r] = sum over column slice t of s (q - z) x'     HBM stream
//   decode_yout  y = S_G^-1 D_out (I (x) H_kout) (sum_t P[t]) / sqrt(kout)
// decode_gemv carries all the weight bytes.  A wave reads 16 bytes of a row per
// lane (one 1 KiB coalesced load per row and slice).  A workgroup issues its x
// loads, then every weight load of its rows, and builds x' in LDS while the
// weights are in flight (a workgroup barrier waits for LDS traffic only).
// Each lane keeps the x' values of its chunk in registers for all its rows.
// Codes stored in processing order (act-order layers) come with the
// permutation: the workgroup then builds the whole x' and gathers x'[perm[c]].
// The zero point is folded out of the inner loop:
// sum s (q - z) x' = s (sum q x' - z sum x') per lane chunk (a chunk never
// straddles a group: groups are multiples of 64 columns).  Both launches are
// ordinary stream work (no host synchronization, no memset), so a caller can
// capture them in a HIP graph.
#include <algorithm>
#include <cmath>
#include <mutex>

#include "kronq_internal.h"
#include "wht_lds.h"

namespace kronq {
namespace {

constexpr int NT = 256;

// ---------------------------------------------------------------- pack / unpack

// stored column j holds code column perm[j] (processing order) when perm is
// given, column j otherwise; an entry of perm outside [0, n) reads column 0
__global__ void pack_kernel(const uint8_t* __restrict__ codes, int64_t m, int64_t n, int64_t ldc,
                            int bits, const int32_t* __restrict__ perm, uint8_t* __restrict__ packed,
                            int64_t ldp, int64_t nb) {
  const int per = 8 / bits;
  const uint32_t mask = (1u << bits) - 1u;
  const int64_t total = m * nb;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / nb, b = i - r * nb;
    uint32_t v = 0;
    for (int t = 0; t < per; ++t) {
      const int64_t j = b * per + t;
      if (j < n) {
        int64_t c = perm ? (int64_t)perm[j] : j;
        c = (c >= 0 && c < n) ? c : 0;
        v |= ((uint32_t)codes[r * ldc + c] & mask) << (bits * t);
      }
    }
    packed[r * ldp + b] = (uint8_t)v;
  }
}

__global__ void unpack_kernel(const uint8_t* __restrict__ packed, int64_t m, int64_t n, int64_t ldp,
                              int bits, uint8_t* __restrict__ codes, int64_t ldc) {
  const int per = 8 / bits;
  const uint32_t mask = (1u << bits) - 1u;
  const int64_t total = m * n;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / n, j = i - r * n;
    const uint32_t byte = packed[r * ldp + j / per];
    codes[r * ldc + j] = (uint8_t)((byte >> (bits * (int)(j % per))) & mask);
  }
}

// ---------------------------------------------------------------- output transform

// y = (WHT_kout(sum_t part[t]) * nrm) * signs / sg over a tile of 2^lg_tile
// rows (whole blocks; the tail of the last tile is zero padding, not stored).
// Thread t owns rows t + NTY * j (coalesced); the factors of its rows and the
// partial sums are loaded first (clamped addresses, rows past m discarded by a
// select).  The row bits above 8 (register index j) are transformed in
// registers, bits 0..7 in LDS.
constexpr int NTY = 256;
constexpr int EMAX = 16;   // elements a thread holds: tiles up to 16 * 256 = 4096 in registers

__global__ void __launch_bounds__(NTY) decode_yout(const float* __restrict__ part, int slices,
                                                   int64_t m, const float* __restrict__ sgn,
                                                   const float* __restrict__ sg, int lg_k,
                                                   int lg_tile, float nrm, float* __restrict__ y) {
  extern __shared__ __align__(16) float s[];
  const int T = 1 << lg_tile;
  const int t = threadIdx.x;
  const int64_t base = (int64_t)blockIdx.x << lg_tile;
  // NULL signs or S_G: the loads read the partial sums (at least m floats)
  // in their place and a select takes 1, so that no load sits behind a branch
  const float* sga = sgn ? sgn : part;
  const float* sgb = sg ? sg : part;
  float v[EMAX], f[EMAX];
#pragma unroll
  for (int j = 0; j < EMAX; ++j) {
    const int64_t r = base + t + NTY * j;
    const bool in = (t + NTY * j < T) && r < m;
    const int64_t rr = in ? r : 0;
    const float a0 = sga[rr], b0 = sgb[rr];
    const float a = sgn ? a0 : 1.f, b = sg ? b0 : 1.f;   // NULL signs: identity side
    f[j] = nrm * a / b;
    v[j] = 0.f;
  }
#pragma unroll 2
  for (int q = 0; q < slices; ++q) {
    const float* pq = part + (int64_t)q * m;
#pragma unroll
    for (int j = 0; j < EMAX; ++j) {
      const int64_t r = base + t + NTY * j;
      const bool in = (t + NTY * j < T) && r < m;
      const float a = pq[in ? r : 0];
      v[j] += in ? a : 0.f;
    }
  }
  const bool regs = T <= EMAX * NTY;
  wht_regs_masked<EMAX>(v, T / NTY, regs ? (1 << min(4, max(0, lg_k - 8))) - 1 : 0);
#pragma unroll
  for (int j = 0; j < EMAX; ++j)
    if (t + NTY * j < T) s[pad(t + NTY * j)] = v[j];
  for (int e = t + NTY * EMAX; e < T; e += NTY) {   // tiles above 4096 rows
    float a = 0.f;
    for (int q = 0; q < slices; ++q)
      if (base + e < m) a += part[(int64_t)q * m + base + e];
    s[pad(e)] = a;
  }
  __syncthreads();
  lds_wht_low_bits<NTY>(s, lg_tile, regs ? min(lg_k, 8) : lg_k);
#pragma unroll
  for (int j = 0; j < EMAX; ++j) {
    const int64_t r = base + t + NTY * j;
    if (t + NTY * j < T && r < m) y[r] = s[pad(t + NTY * j)] * f[j];
  }
  for (int e = t + NTY * EMAX; e < T; e += NTY) {
    const int64_t r = base + e;
    if (r < m) y[r] = s[pad(e)] * (nrm * (sgn ? sgn[r] : 1.f) / (sg ? sg[r] : 1.f));
  }
}

// ---------------------------------------------------------------- dequantizing matvec

struct GemvParams {
  const uint8_t* codes;
  int64_t ldp;          // bytes per stored row (multiple of 16)
  int64_t nbytes;       // bytes of a row that hold codes
  const float* scales;
  const float* zeros;
  int64_t ngroups;
  int64_t group;        // 0: one grid per row
  const float* x;       // input vector (n)
  const float* sgn_in;  // D_in (n)
  const int32_t* perm;  // stored column j is natural column perm[j] (NULL: natural order)
  int lg_kin;           // log2 of the input block
  int lg_tile;          // log2 of the x' tile: max(slice width, input block)
  float nrm_in;         // 1 / sqrt(kin)
  int64_t m, n;
  int slices;
  float* part;          // slices x m partial sums
};

template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float dpp_add(float v) {
  // lanes the DPP source leaves out (rows outside ROWS) add 0
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                   CTRL, ROWS, 0xF, false));
}

// Sum over the 64 lanes, returned as a wave-uniform value: butterflies within
// quads and rows of 16 (quad_perm, half-mirror, mirror), then lane 15 of each
// row into the next row and lane 31 into the upper half (row broadcasts); lane
// 63 ends with the total.  All VALU data movement, no LDS round trips.
__device__ __forceinline__ float wave_total(float v) {
  v = dpp_add<0xB1>(v);         // quad_perm [1,0,3,2]
  v = dpp_add<0x4E>(v);         // quad_perm [2,3,0,1]
  v = dpp_add<0x141>(v);        // row_half_mirror
  v = dpp_add<0x140>(v);        // row_mirror: every lane holds its row's sum
  v = dpp_add<0x142, 0xA>(v);   // row_bcast15 into rows 1 and 3
  v = dpp_add<0x143, 0xC>(v);   // row_bcast31 into rows 2 and 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// sum over the lane's 16 bytes of code * x' (one code a byte for BITS 8; for
// BITS 2 and 4, 8 / BITS codes a byte, low bits first).  Codes of 2 and 4 bits
// are spread one a byte and converted two at a time as fp8 e4m3: a byte value
// c < 16 has exponent field 0 or 1, where the format is linear, so it decodes
// to exactly c * unit (unit = the value of byte 1, a power of two); the caller
// multiplies the sum by 1 / unit.
template <int BITS>
__device__ __forceinline__ float chunk_dot(const uint4& q, const float* xr) {
  constexpr int PER = 8 / BITS;
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  float acc0 = 0.f, acc1 = 0.f;
  if constexpr (BITS == 8) {
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float c = (float)((w[d] >> (8 * k)) & 0xFFu);
        if (k & 1) acc1 = fmaf(c, xr[4 * d + k], acc1);
        else acc0 = fmaf(c, xr[4 * d + k], acc0);
      }
  } else {
    constexpr uint32_t MASK = ((1u << BITS) - 1u) * 0x01010101u;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int t = 0; t < PER; ++t) {
        const uint32_t b = (w[d] >> (BITS * t)) & MASK;   // byte k holds code 4*PER*d + PER*k + t
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)b, false);   // bytes 0, 1
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)b, true);    // bytes 2, 3
        const float* xp = xr + 4 * PER * d + t;
        acc0 = fmaf(lo[0], xp[0], acc0);
        acc1 = fmaf(lo[1], xp[PER], acc1);
        acc0 = fmaf(hi[0], xp[2 * PER], acc0);
        acc1 = fmaf(hi[1], xp[3 * PER], acc1);
      }
  }
  return acc0 + acc1;
}

// One workgroup: column slice sl (SW columns) x 4U rows.  x' of the slice is
// built here: x * D_in through the input butterflies in LDS over a tile of
// max(SW, kin) columns (a block wider than the slice is transformed whole and
// the slice kept).
template <int BITS, int U, bool GROUPED>
__global__ void __launch_bounds__(NT) decode_gemv(GemvParams p) {
  constexpr int CPL = (BITS == 8) ? 16 : 128 / BITS;   // codes a lane holds per row (16 bytes)
  constexpr int SW = 64 * CPL;                        // columns per slice
  extern __shared__ __align__(16) float tile[];
  const int sl = (int)(blockIdx.x % (unsigned)p.slices);
  const int64_t rg = blockIdx.x / (unsigned)p.slices;
  const int64_t c0 = (int64_t)sl * SW;
  const int T = 1 << p.lg_tile;                       // >= SW >= 1024
  const int64_t tb = (c0 >> p.lg_tile) << p.lg_tile;  // first column of the tile
  const int off = (int)(c0 - tb);
  const int ept = T / NT;                             // tile elements a thread holds (>= 4)
  const int t = threadIdx.x;

  // Loads below read clamped, always valid addresses and discard what lies
  // outside the matrix with a select, so they issue back to back.
  // 1. x and D_in: thread t holds tile elements t + NT * j (coalesced)
  // NULL signs (identity side): the loads read x in their place and a select
  // takes 1, so that no load sits behind a branch
  const float* sgi = p.sgn_in ? p.sgn_in : p.x;
  float xv[EMAX], sv[EMAX];
#pragma unroll
  for (int j = 0; j < EMAX; ++j) {
    const int64_t c = tb + t + NT * j;
    const bool in = (j < ept) && (c < p.n);
    const int64_t cc = in ? c : 0;
    const float a = p.x[cc], b0 = sgi[cc];
    const float b = p.sgn_in ? b0 : 1.f;
    xv[j] = in ? a : 0.f;
    sv[j] = in ? b : 0.f;
  }

  // 2. weight rows and their grids
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t lane_b = (int64_t)sl * 1024 + lane * 16;   // first byte of the lane's chunk
  const bool live = lane_b < p.nbytes;                      // then lane_b + 16 <= ldp
  const int64_t lb = live ? lane_b : 0;
  // grouped: the chunk lies in one group (group % 64 == 0, n % group == 0)
  const int64_t g = (GROUPED && live) ? (int64_t)((uint32_t)(c0 + lane * CPL) / (uint32_t)p.group) : 0;
  const int64_t r0 = rg * (4 * U) + wave * U;
  uint4 q[U];
  float sc[U], zr[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t r = r0 + u;
    const bool rin = r < p.m;
    const int64_t rr = rin ? r : 0;
    const uint4 v = *reinterpret_cast<const uint4*>(p.codes + rr * p.ldp + lb);
    const bool use = rin && live;
    q[u] = make_uint4(use ? v.x : 0u, use ? v.y : 0u, use ? v.z : 0u, use ? v.w : 0u);
    const float a = p.scales[rr * p.ngroups + g], b = p.zeros[rr * p.ngroups + g];
    sc[u] = rin ? a : 0.f;
    zr[u] = rin ? b : 0.f;
  }

  // 3. x' = WHT(x * D_in): element bits 8.. (register index j) in registers
  //    when they lie inside an input block, bits below 8 in LDS; tiles above
  //    EMAX * NT columns load the rest here and run every bit in LDS
  const bool regs = ept <= EMAX;
#pragma unroll
  for (int j = 0; j < EMAX; ++j) xv[j] *= sv[j];
  wht_regs_masked<EMAX>(xv, ept, regs ? (1 << min(4, max(0, p.lg_kin - 8))) - 1 : 0);
#pragma unroll
  for (int j = 0; j < EMAX; ++j)
    if (j < ept) tile[pad(t + NT * j)] = xv[j];
  for (int j = EMAX; j < ept; ++j) {
    const int e = t + NT * j;
    const int64_t ce = (tb + e < p.n) ? tb + e : 0;
    const float a = p.x[ce], b0 = sgi[ce];
    tile[pad(e)] = (tb + e < p.n) ? a * (p.sgn_in ? b0 : 1.f) : 0.f;
  }
  __syncthreads();
  lds_wht_low_bits<NT>(tile, p.lg_tile, regs ? min(p.lg_kin, 8) : p.lg_kin);
  float xr[CPL];
  if (p.perm) {
    // codes stored in processing order: the tile holds the whole x' and the
    // lane gathers x'[perm[c]] for its stored columns c (clamped into [0, n))
    const int64_t cb = c0 + lane * CPL;
    int pi[CPL];
#pragma unroll
    for (int k = 0; k < CPL; ++k) pi[k] = p.perm[cb + k < p.n ? cb + k : 0];
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      const int c = min(max(pi[k], 0), (int)p.n - 1);
      xr[k] = (cb + k < p.n) ? tile[pad(c)] * p.nrm_in : 0.f;
    }
  } else {
#pragma unroll
    for (int k = 0; k < CPL; k += 4) {
      const float4 v = *reinterpret_cast<const float4*>(tile + pad(off + lane * CPL + k));
      xr[k] = v.x * p.nrm_in;
      xr[k + 1] = v.y * p.nrm_in;
      xr[k + 2] = v.z * p.nrm_in;
      xr[k + 3] = v.w * p.nrm_in;
    }
  }
  float xsum = 0.f;
#pragma unroll
  for (int k = 0; k < CPL; ++k) xsum += xr[k];
  const float xtot = GROUPED ? 0.f : wave_total(xsum);

  // 4. dequantized dot products, zero point folded out of the inner loop;
  //    lane u stores row u
  float out = 0.f;
  const float unit_inv =
      (BITS == 8) ? 1.f : 1.f / __builtin_amdgcn_cvt_pk_f32_fp8(1, false)[0];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const float a = chunk_dot<BITS>(q[u], xr) * unit_inv;
    float v;
    if (GROUPED) {
      v = wave_total(live ? sc[u] * (a - zr[u] * xsum) : 0.f);
    } else {
      v = sc[u] * (wave_total(a) - zr[u] * xtot);
    }
    out = (lane == u) ? v : out;
  }
  if (lane < U && r0 + lane < p.m) p.part[(int64_t)sl * p.m + r0 + lane] = out;
}

int ilog2(int64_t x) {
  int l = 0;
  while ((int64_t(1) << l) < x) ++l;
  return l;
}

int codes_per_lane(int bits) { return (bits == 2 || bits == 4) ? 128 / bits : 16; }

int64_t slices_of(int64_t n, int bits) {
  const int64_t sw = 64 * codes_per_lane(bits);
  return (n + sw - 1) / sw;
}

kronq_status set_lds(const void* fn, size_t bytes) {
  if (bytes > 65536)
    KQ_HIP(hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes));
  return KRONQ_OK;
}

template <int BITS, bool GROUPED>
kronq_status gemv_dispatch(const GemvParams& p, hipStream_t st) {
  const int64_t S = p.slices;
  // about one workgroup per CU or more: rows per workgroup 32, 16 or 8
  int U = 2;
  if (S * ((p.m + 31) / 32) >= 256) U = 8;
  else if (S * ((p.m + 15) / 16) >= 256) U = 4;
  const int64_t rows_per_wg = 4 * U;
  const int64_t grid = S * ((p.m + rows_per_wg - 1) / rows_per_wg);
  if (grid > 0x7fffffff) return fail(KRONQ_EINVAL, "decode_gemv: grid too large");
  const size_t lds = (size_t)padded(1 << p.lg_tile) * sizeof(float);
  const void* fn = U == 8 ? (const void*)decode_gemv<BITS, 8, GROUPED>
                 : U == 4 ? (const void*)decode_gemv<BITS, 4, GROUPED>
                          : (const void*)decode_gemv<BITS, 2, GROUPED>;
  kronq_status s = set_lds(fn, lds);
  if (s) return s;
  switch (U) {
    case 8: hipLaunchKernelGGL((decode_gemv<BITS, 8, GROUPED>), dim3((unsigned)grid), dim3(NT), lds, st, p); break;
    case 4: hipLaunchKernelGGL((decode_gemv<BITS, 4, GROUPED>), dim3((unsigned)grid), dim3(NT), lds, st, p); break;
    default: hipLaunchKernelGGL((decode_gemv<BITS, 2, GROUPED>), dim3((unsigned)grid), dim3(NT), lds, st, p); break;
  }
  KQ_LAUNCHED("decode_gemv");
  return KRONQ_OK;
}

template <int BITS>
kronq_status gemv_bits(const GemvParams& p, hipStream_t st) {
  return p.group > 0 ? gemv_dispatch<BITS, true>(p, st) : gemv_dispatch<BITS, false>(p, st);
}

}  // namespace

kronq_status pack_launch(const uint8_t* codes, int64_t m, int64_t n, int64_t ldc, int bits,
                         const int32_t* perm, uint8_t* packed, int64_t ldp, hipStream_t s) {
  const int64_t nb = (n * bits + 7) / 8;
  const int64_t total = m * nb;
  const int64_t grid = std::min<int64_t>((total + 255) / 256, 65536);
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)grid), dim3(256), 0, s, codes, m, n, ldc, bits,
                     perm, packed, ldp, nb);
  KQ_LAUNCHED("pack_kernel");
  return KRONQ_OK;
}

kronq_status unpack_launch(const uint8_t* packed, int64_t m, int64_t n, int64_t ldp, int bits,
                           uint8_t* codes, int64_t ldc, hipStream_t s) {
  const int64_t total = m * n;
  const int64_t grid = std::min<int64_t>((total + 255) / 256, 65536);
  hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)grid), dim3(256), 0, s, packed, m, n, ldp,
                     bits, codes, ldc);
  KQ_LAUNCHED("unpack_kernel");
  return KRONQ_OK;
}

int64_t decode_row_bytes(int64_t n, int bits) {
  return (bits == 2 || bits == 4) ? (n * bits + 7) / 8 : n;
}

size_t decode_ws_bytes(int64_t m, int64_t n, int bits) {
  return align_up((size_t)slices_of(n, bits) * (size_t)m * sizeof(float), 256);
}

kronq_status decode_launch(const uint8_t* codes, int64_t m, int64_t n, int64_t ldp, int bits,
                           int64_t group, const float* scales, const float* zeros,
                           const int32_t* perm, const kronq_had& in, const kronq_had& out,
                           const float* sg, const float* x, float* y, void* ws, hipStream_t s) {
  // partial row sums of W^ x', with x' = V x built per workgroup
  GemvParams p{};
  p.codes = codes;
  p.ldp = ldp;
  p.nbytes = decode_row_bytes(n, bits);
  p.scales = scales;
  p.zeros = zeros;
  p.group = group;
  p.ngroups = group > 0 ? n / group : 1;
  p.x = x;
  p.sgn_in = in.signs;
  p.lg_kin = ilog2(in.block);
  p.lg_tile = std::max(ilog2(64 * codes_per_lane(bits)), p.lg_kin);
  p.perm = perm;
  if (perm) p.lg_tile = std::max(p.lg_tile, ilog2(n));   // the whole x' in one tile
  p.nrm_in = (float)(1.0 / std::sqrt((double)in.block));
  p.m = m;
  p.n = n;
  p.slices = (int)slices_of(n, bits);
  p.part = static_cast<float*>(ws);
  kronq_status st = (bits == 4) ? gemv_bits<4>(p, s)
                   : (bits == 2) ? gemv_bits<2>(p, s)
                                 : gemv_bits<8>(p, s);
  if (st) return st;
  // y = S_G^-1 U^T y'  (tiles of max(kout, min(4096, m)) rows)
  const int lg_k = ilog2(out.block);
  const int lg_t = std::max(lg_k, std::min(12, ilog2(m)));
  const int64_t tiles = (m + (int64_t(1) << lg_t) - 1) >> lg_t;
  const size_t lds = (size_t)padded(1 << lg_t) * sizeof(float);
  st = set_lds((const void*)decode_yout, lds);
  if (st) return st;
  hipLaunchKernelGGL(decode_yout, dim3((unsigned)tiles), dim3(NTY), lds, s, p.part, p.slices, m,
                     out.signs, sg, lg_k, lg_t, (float)(1.0 / std::sqrt((double)out.block)), y);
  KQ_LAUNCHED("decode_yout");
  return KRONQ_OK;
}

// ------------------------------------------------- decode without allocation
//
// For callers that cannot allocate (code under HIP graph capture, serving
// loops, harnesses that forbid hipMalloc): the slice partial sums live in a
// fixed device array of this module, one copy per GPU, held until the process
// ends.  On the host the array's name is only a stand-in for the symbol; its
// device address is looked up once per device (with that device current) and
// only that address is handed to kernels.  Every call on a GPU shares the
// GPU's copy: calls that overlap on one GPU race on it.  The partial sums are
// written in full before they are read, so nothing needs clearing.

constexpr size_t kDecodeScratchBytes = size_t(4) << 20;   // 4 MiB: 2^20 partial sums

static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// device address of `scratch` on the calling thread's current device
kronq_status scratch_address(void** out) {
  int dev = -1;
  KQ_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(KRONQ_EUNSUPPORTED, "decode scratch: device %d outside 0..%d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(decode scratch)");
    if (!p) return fail(KRONQ_EHIP, "hipGetSymbolAddress(decode scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KRONQ_OK;
}

}  // namespace

size_t decode_scratch_bytes() { return kDecodeScratchBytes; }

kronq_status decode_launch_noalloc(const uint8_t* codes, int64_t m, int64_t n, int64_t ldp, int bits,
                                   int64_t group, const float* scales, const float* zeros,
                                   const int32_t* perm, const kronq_had& in, const kronq_had& out,
                                   const float* sg, const float* x, float* y, hipStream_t s) {
  const size_t need = decode_ws_bytes(m, n, bits);
  if (need > kDecodeScratchBytes)
    return fail(KRONQ_ENOMEM, "kronq_decode_matvec_noalloc: %zu bytes of partial sums exceed the "
                "fixed %zu-byte buffer", need, kDecodeScratchBytes);
  void* ws = nullptr;
  const kronq_status st = scratch_address(&ws);
  if (st) return st;
  return decode_launch(codes, m, n, ldp, bits, group, scales, zeros, perm, in, out, sg, x, y, ws, s);
}

}  // namespace kronq
