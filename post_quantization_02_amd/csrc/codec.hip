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
// Decode of y = S_G^-1 U^T W^ V x with W^[r][c] = s[r][g] (q[r][c] - z[r][g]):
//   decode_xin  x' = V x = (I (x) H_kin) D_in x / sqrt(kin)        LDS butterflies
//   decode_gemv P[t][r] = sum over column slice t of s (q - z) x'   HBM stream
//   decode_yout y = S_G^-1 D_out (I (x) H_kout) (sum_t P[t]) / sqrt(kout)
// decode_gemv carries all the weight bytes.  A wave reads 16 bytes of a row per
// lane (one 1 KiB coalesced load per row and slice) and keeps the x' values
// of its chunk in registers for every row it visits, so x' costs no LDS or
// cache traffic per row.  The zero point is folded out of the inner
// loop: sum s (q - z) x' = s (sum q x' - z sum x') per lane chunk (a chunk
// never straddles a group: groups are multiples of 64 columns).  The three
// launches are ordinary stream work (no host synchronization, no memset), so
// a caller can capture them in a HIP graph.
#include <algorithm>
#include <cmath>

#include "kronq_internal.h"
#include "wht_lds.h"

namespace kronq {
namespace {

constexpr int NT = 256;
constexpr int kLgTileVec = 13;   // vector transform tile: 8192 floats unless a block is longer

// ---------------------------------------------------------------- pack / unpack

__global__ void pack_kernel(const uint8_t* __restrict__ codes, int64_t m, int64_t n, int64_t ldc,
                            int bits, uint8_t* __restrict__ packed, int64_t ldp, int64_t nb) {
  const int per = 8 / bits;
  const uint32_t mask = (1u << bits) - 1u;
  const int64_t total = m * nb;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / nb, b = i - r * nb;
    uint32_t v = 0;
    for (int t = 0; t < per; ++t) {
      const int64_t j = b * per + t;
      if (j < n) v |= ((uint32_t)codes[r * ldc + j] & mask) << (bits * t);
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

// ---------------------------------------------------------------- vector transforms

// x' = WHT_kin(x * signs) * nrm over a tile of 2^lg_tile elements (whole blocks;
// the tail of the last tile is zero padding and is not stored)
__global__ void __launch_bounds__(NT) decode_xin(const float* __restrict__ x,
                                                 const float* __restrict__ sgn, int64_t n,
                                                 int lg_k, int lg_tile, float nrm,
                                                 float* __restrict__ xp) {
  extern __shared__ __align__(16) float s[];
  const int T = 1 << lg_tile;
  const int64_t base = (int64_t)blockIdx.x << lg_tile;
  for (int e = threadIdx.x; e < T; e += NT) {
    const int64_t i = base + e;
    s[pad(e)] = (i < n) ? x[i] * sgn[i] : 0.f;
  }
  __syncthreads();
  lds_wht_bits<NT>(s, lg_tile, 0, lg_k);
  for (int e = threadIdx.x; e < T; e += NT) {
    const int64_t i = base + e;
    if (i < n) xp[i] = s[pad(e)] * nrm;
  }
}

// y = (WHT_kout(sum_t part[t]) * nrm) * signs / sg
__global__ void __launch_bounds__(NT) decode_yout(const float* __restrict__ part, int slices,
                                                  int64_t m, const float* __restrict__ sgn,
                                                  const float* __restrict__ sg, int lg_k,
                                                  int lg_tile, float nrm, float* __restrict__ y) {
  extern __shared__ __align__(16) float s[];
  const int T = 1 << lg_tile;
  const int64_t base = (int64_t)blockIdx.x << lg_tile;
  for (int e = threadIdx.x; e < T; e += NT) {
    const int64_t i = base + e;
    float v = 0.f;
    if (i < m)
      for (int t = 0; t < slices; ++t) v += part[(int64_t)t * m + i];
    s[pad(e)] = v;
  }
  __syncthreads();
  lds_wht_bits<NT>(s, lg_tile, 0, lg_k);
  for (int e = threadIdx.x; e < T; e += NT) {
    const int64_t i = base + e;
    if (i < m) {
      const float f = sg ? sgn[i] / sg[i] : sgn[i];
      y[i] = s[pad(e)] * nrm * f;
    }
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
  const float* xp;
  int64_t m, n;
  int slices;
  float* part;          // slices x m partial sums
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// sum over the lane's 16 bytes of code * x'  (BITS 2 or 4: 8/BITS codes a byte,
// low bits first; BITS 8: one code a byte)
template <int BITS>
__device__ __forceinline__ float chunk_dot(const uint4& q, const float* xr) {
  constexpr int PER = 8 / BITS;
  constexpr uint32_t MASK = (BITS == 8) ? 0xFFFFFFFFu
                                        : ((1u << BITS) - 1u) * 0x01010101u;
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int t = 0; t < PER; ++t) {
      const uint32_t b = (w[d] >> (BITS * t)) & MASK;   // byte k holds code 4*PER*d + PER*k + t
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float c = (float)((b >> (8 * k)) & 0xFFu);
        const float xv = xr[4 * PER * d + PER * k + t];
        if (k & 1) acc1 = fmaf(c, xv, acc1);
        else acc0 = fmaf(c, xv, acc0);
      }
    }
  return acc0 + acc1;
}

template <int BITS, int U>
__global__ void __launch_bounds__(NT) decode_gemv(GemvParams p) {
  constexpr int CPL = (BITS == 8) ? 16 : 128 / BITS;   // codes a lane holds per row (16 bytes)
  constexpr int SW = 64 * CPL;                        // columns per slice
  __shared__ __align__(16) float xs[SW];
  const int sl = (int)(blockIdx.x % (unsigned)p.slices);
  const int64_t rg = blockIdx.x / (unsigned)p.slices;
  const int64_t c0 = (int64_t)sl * SW;
  for (int i = threadIdx.x; i < SW; i += NT) xs[i] = (c0 + i < p.n) ? p.xp[c0 + i] : 0.f;
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  float xr[CPL];
#pragma unroll
  for (int k = 0; k < CPL; k += 4) {
    const float4 v = *reinterpret_cast<const float4*>(xs + lane * CPL + k);
    xr[k] = v.x;
    xr[k + 1] = v.y;
    xr[k + 2] = v.z;
    xr[k + 3] = v.w;
  }
  float xsum = 0.f;
#pragma unroll
  for (int k = 0; k < CPL; ++k) xsum += xr[k];

  const int64_t lane_b = (int64_t)sl * 1024 + lane * 16;   // first byte of the lane's chunk
  const bool live = lane_b < p.nbytes;                      // then lane_b + 16 <= ldp
  const bool grouped = p.group > 0;
  // grouped: the chunk lies in one group (group % 64 == 0, n % group == 0)
  const int64_t g = (grouped && live) ? (c0 + lane * CPL) / p.group : 0;
  const float xtot = grouped ? 0.f : wave_sum(xsum);

  const int64_t r0 = rg * (4 * U) + wave * U;
  uint4 q[U];
  float sc[U], zr[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t r = r0 + u;
    q[u] = make_uint4(0u, 0u, 0u, 0u);
    sc[u] = 0.f;
    zr[u] = 0.f;
    if (r < p.m) {
      if (live) q[u] = *reinterpret_cast<const uint4*>(p.codes + r * p.ldp + lane_b);
      if (grouped) {
        if (live) {
          sc[u] = p.scales[r * p.ngroups + g];
          zr[u] = p.zeros[r * p.ngroups + g];
        }
      } else {
        sc[u] = p.scales[r * p.ngroups];
        zr[u] = p.zeros[r * p.ngroups];
      }
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t r = r0 + u;
    const float a = chunk_dot<BITS>(q[u], xr);
    float v;
    if (grouped) {
      v = wave_sum(sc[u] * (a - zr[u] * xsum));
    } else {
      v = sc[u] * (wave_sum(a) - zr[u] * xtot);
    }
    if (lane == 0 && r < p.m) p.part[(int64_t)sl * p.m + r] = v;
  }
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

template <int BITS>
kronq_status gemv_dispatch(const GemvParams& p, hipStream_t st) {
  const int64_t S = p.slices;
  const int64_t target = 512;   // two workgroups per CU
  int U = 2;
  if (S * ((p.m + 31) / 32) >= target) U = 8;
  else if (S * ((p.m + 15) / 16) >= target) U = 4;
  const int64_t rows_per_wg = 4 * U;
  const int64_t grid = S * ((p.m + rows_per_wg - 1) / rows_per_wg);
  if (grid > 0x7fffffff) return fail(KRONQ_EINVAL, "decode_gemv: grid too large");
  switch (U) {
    case 8: hipLaunchKernelGGL((decode_gemv<BITS, 8>), dim3((unsigned)grid), dim3(NT), 0, st, p); break;
    case 4: hipLaunchKernelGGL((decode_gemv<BITS, 4>), dim3((unsigned)grid), dim3(NT), 0, st, p); break;
    default: hipLaunchKernelGGL((decode_gemv<BITS, 2>), dim3((unsigned)grid), dim3(NT), 0, st, p); break;
  }
  KQ_LAUNCHED("decode_gemv");
  return KRONQ_OK;
}

// tile of the vector transforms: whole blocks, at least one block, at most
// max(block, 2^kLgTileVec) elements and no longer than the vector needs
int vec_tile_lg(int64_t len, int lg_k) {
  const int lg_len = ilog2(len);
  int lg = std::min(kLgTileVec, lg_len);
  return std::max(lg, lg_k);
}

kronq_status set_lds(const void* fn, size_t bytes) {
  if (bytes > 65536)
    KQ_HIP(hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes));
  return KRONQ_OK;
}

}  // namespace

kronq_status pack_launch(const uint8_t* codes, int64_t m, int64_t n, int64_t ldc, int bits,
                         uint8_t* packed, int64_t ldp, hipStream_t s) {
  const int64_t nb = (n * bits + 7) / 8;
  const int64_t total = m * nb;
  const int64_t grid = std::min<int64_t>((total + 255) / 256, 65536);
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)grid), dim3(256), 0, s, codes, m, n, ldc, bits,
                     packed, ldp, nb);
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
  return align_up((size_t)n * sizeof(float), 256) +
         align_up((size_t)slices_of(n, bits) * (size_t)m * sizeof(float), 256);
}

kronq_status decode_launch(const uint8_t* codes, int64_t m, int64_t n, int64_t ldp, int bits,
                           int64_t group, const float* scales, const float* zeros,
                           const kronq_had& in, const kronq_had& out, const float* sg,
                           const float* x, float* y, void* ws, hipStream_t s) {
  float* xp = static_cast<float*>(ws);
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                         align_up((size_t)n * sizeof(float), 256));
  // x' = V x
  {
    const int lg_k = ilog2(in.block);
    const int lg_t = vec_tile_lg(n, lg_k);
    const int64_t tiles = (n + (int64_t(1) << lg_t) - 1) >> lg_t;
    const size_t lds = (size_t)padded(1 << lg_t) * sizeof(float);
    kronq_status st = set_lds((const void*)decode_xin, lds);
    if (st) return st;
    hipLaunchKernelGGL(decode_xin, dim3((unsigned)tiles), dim3(NT), lds, s, x, in.signs, n, lg_k,
                       lg_t, (float)(1.0 / std::sqrt((double)in.block)), xp);
    KQ_LAUNCHED("decode_xin");
  }
  // partial row sums of W^ x'
  GemvParams p{};
  p.codes = codes;
  p.ldp = ldp;
  p.nbytes = decode_row_bytes(n, bits);
  p.scales = scales;
  p.zeros = zeros;
  p.group = group;
  p.ngroups = group > 0 ? n / group : 1;
  p.xp = xp;
  p.m = m;
  p.n = n;
  p.slices = (int)slices_of(n, bits);
  p.part = part;
  kronq_status st = (bits == 4) ? gemv_dispatch<4>(p, s)
                   : (bits == 2) ? gemv_dispatch<2>(p, s)
                                 : gemv_dispatch<8>(p, s);
  if (st) return st;
  // y = S_G^-1 U^T y'
  {
    const int lg_k = ilog2(out.block);
    const int lg_t = vec_tile_lg(m, lg_k);
    const int64_t tiles = (m + (int64_t(1) << lg_t) - 1) >> lg_t;
    const size_t lds = (size_t)padded(1 << lg_t) * sizeof(float);
    st = set_lds((const void*)decode_yout, lds);
    if (st) return st;
    hipLaunchKernelGGL(decode_yout, dim3((unsigned)tiles), dim3(NT), lds, s, part, p.slices, m,
                       out.signs, sg, lg_k, lg_t, (float)(1.0 / std::sqrt((double)out.block)), y);
    KQ_LAUNCHED("decode_yout");
  }
  return KRONQ_OK;
}

}  // namespace kronq
