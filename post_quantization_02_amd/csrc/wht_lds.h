// Walsh-Hadamard butterflies on a tile staged in LDS (Sylvester order, no
// normalization), shared by the incoherence transforms and the deploy decode.
//
// A tile holds 2^p floats; index bits [blo, bhi) are transformed, the other bits
// select independent vectors.  Rounds of up to 4 bits: a thread gathers the 16
// elements that differ in those bits, runs 4 butterfly stages in registers and
// scatters them back.  Rows of 32 floats are padded by 4 so float4-aligned
// accesses stay 16-byte aligned and the low-bit rounds are bank-conflict free.
#pragma once

#include <hip/hip_runtime.h>

namespace kronq {

__host__ __device__ constexpr int pad(int i) { return i + ((i >> 5) << 2); }
constexpr int padded(int n) { return n + ((n >> 5) << 2); }

// In-register Walsh-Hadamard over K bits (2^K values, natural order).
template <int K>
__device__ __forceinline__ void wht_regs(float (&v)[1 << K]) {
#pragma unroll
  for (int h = 1; h < (1 << K); h <<= 1)
#pragma unroll
    for (int i = 0; i < (1 << K); ++i)
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
}

template <int NT, int K>
__device__ __forceinline__ void lds_round(float* s, int p, int b) {
  const int ngroups = 1 << (p - K);
  const int lowmask = (1 << b) - 1;
  for (int g = threadIdx.x; g < ngroups; g += NT) {
    const int base = ((g >> b) << (b + K)) | (g & lowmask);
    float v[1 << K];
#pragma unroll
    for (int c = 0; c < (1 << K); ++c) v[c] = s[pad(base | (c << b))];
    wht_regs<K>(v);
#pragma unroll
    for (int c = 0; c < (1 << K); ++c) s[pad(base | (c << b))] = v[c];
  }
}

// Unnormalized WHT over index bits [blo, bhi) of the 2^p-element LDS tile
// (NT threads; every thread of the workgroup must call it).
template <int NT>
__device__ void lds_wht_bits(float* s, int p, int blo, int bhi) {
  for (int b = blo; b < bhi; b += 4) {
    const int k = min(4, bhi - b);
    switch (k) {
      case 4: lds_round<NT, 4>(s, p, b); break;
      case 3: lds_round<NT, 3>(s, p, b); break;
      case 2: lds_round<NT, 2>(s, p, b); break;
      default: lds_round<NT, 1>(s, p, b); break;
    }
    __syncthreads();
  }
}

// Rounds at compile-time bit positions.  For indices with disjoint bits,
// pad(a | b) = pad(a) + pad(b), so the 2^K elements of a butterfly group sit
// at constant offsets pad(c << B) from pad(base): the LDS accesses take
// immediate offsets and a group costs one address computation.
template <int NT, int K, int B>
__device__ __forceinline__ void lds_round_cb(float* s, int p) {
  const int ngroups = 1 << (p - K);
  constexpr int lowmask = (1 << B) - 1;
  for (int g = threadIdx.x; g < ngroups; g += NT) {
    float* sb = s + pad(((g >> B) << (B + K)) | (g & lowmask));
    float v[1 << K];
#pragma unroll
    for (int c = 0; c < (1 << K); ++c) v[c] = sb[pad(c << B)];
    wht_regs<K>(v);
#pragma unroll
    for (int c = 0; c < (1 << K); ++c) sb[pad(c << B)] = v[c];
  }
}

template <int NT, int B>
__device__ __forceinline__ void lds_round_k(float* s, int p, int k) {
  switch (k) {
    case 4: lds_round_cb<NT, 4, B>(s, p); break;
    case 3: lds_round_cb<NT, 3, B>(s, p); break;
    case 2: lds_round_cb<NT, 2, B>(s, p); break;
    default: lds_round_cb<NT, 1, B>(s, p); break;
  }
}

// Unnormalized WHT over index bits [0, bhi) of the 2^p-element LDS tile
// (bhi <= 16), rounds of 4 bits at compile-time positions; every thread of
// the workgroup must call it.  Ends with a barrier when it ran a round.
template <int NT>
__device__ __forceinline__ void lds_wht_low_bits(float* s, int p, int bhi) {
  if (bhi > 0) { lds_round_k<NT, 0>(s, p, min(4, bhi)); __syncthreads(); }
  if (bhi > 4) { lds_round_k<NT, 4>(s, p, min(4, bhi - 4)); __syncthreads(); }
  if (bhi > 8) { lds_round_k<NT, 8>(s, p, min(4, bhi - 8)); __syncthreads(); }
  if (bhi > 12) { lds_round_k<NT, 12>(s, p, min(4, bhi - 12)); __syncthreads(); }
}

// WHT over the index bits held in registers: v[j] is element base + stride * j;
// stage h (j-bit log2 h) runs when h < n and the bit is inside the block
// (stage mask bit log2 h set).  Stages are uniform branches, no dynamic indexing.
template <int E>
__device__ __forceinline__ void wht_regs_masked(float (&v)[E], int n, int stage_mask) {
#pragma unroll
  for (int lh = 0; (1 << lh) < E; ++lh) {
    const int h = 1 << lh;
    if (h < n && ((stage_mask >> lh) & 1)) {
#pragma unroll
      for (int i = 0; i < E; ++i)
        if ((i & h) == 0) {
          const float a = v[i], b = v[i + h];
          v[i] = a + b;
          v[i + h] = a - b;
        }
    }
  }
}

}  // namespace kronq
