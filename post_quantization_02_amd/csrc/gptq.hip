// Column-wise OBS quantize-and-compensate with H_X alone (Pith review of the
// KronQ paper, Proposition 1: with H = H_X (x) H_G the column update does not
// depend on H_G, so every output row is an independent GPTQ/GPTAQ problem;
// Algorithm 2: lazy batches of B = 128 columns).
//
// One workgroup owns RT = 16 rows and walks all n columns (processing order)
// in blocks of 128, left-looking, in a single launch:
//   1. acc = W[:, block] - E[:, 0:jb] R[0:jb, block]   (all earlier errors at
//      once; fp64 v_mfma_f64_16x16x4f64, K split over the four waves and
//      reduced in LDS; E is the fp64 error matrix of this workgroup's rows)
//   2. the 128 columns of the block sequentially: each of the four waves owns
//      four rows with 16 lanes per row and 8 columns per lane; the owner lane
//      of column c rounds it onto the grid, forms e = (w - wq) / R[c][c], the
//      error is broadcast across the row's lanes and every later column of the
//      block is compensated with the row of R staged in LDS.
// The loop runs in fp64 from fp32 inputs, so rounding decisions match a
// float64 reference up to summation order.  Grid parameters: per-channel from
// the whole initial row (a separate pass), or per group of g | 128 columns from
// the current compensated values when the group's first column is reached.
#include <utility>

#include "kronq_internal.h"

namespace kronq {
namespace {

typedef double f64x4_t __attribute__((__vector_size__(4 * sizeof(double))));
typedef double f64x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int RT = 16;         // rows per workgroup
constexpr int BLK = 128;       // columns per block
constexpr int GT = 256;        // threads
constexpr int RLD = BLK + 4;   // LDS stride of the R block (floats)

struct GptqParams {
  const float* W;
  int64_t m, n, ldw;
  const float* R;
  int64_t ldr;
  const int32_t* perm;     // may be NULL
  int bits, group;         // group 0: per-channel
  int ngroups;
  uint8_t* codes;
  float* scales;
  float* zeros;
  float* What;             // may be NULL
  float* pre;              // may be NULL
  double* E;               // m x ldE, processing order
  int64_t ldE;             // n rounded up to 16 (128-byte rows)
  const double* pc;        // per-channel (scale, zero) pairs, m x 2
};

// value of `x` held by lane 16 * (lane / 16) + O, for every lane: DPP
// row_newbcast (lane O of each 16-lane row to the whole row), a 64-bit value
// moved as two halves
template <int O>
__device__ __forceinline__ double bcast_row(double x) {
  const long long b = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)b, 0x150 + O, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), 0x150 + O, 0xf, 0xf, false);
  return __longlong_as_double(((long long)(unsigned)hi << 32) | (unsigned)lo);
}

__device__ __forceinline__ int64_t colmap(const GptqParams& p, int64_t j) {
  return p.perm ? (int64_t)p.perm[j] : j;
}

// grid parameters of an asymmetric uniform grid from (min, max)
__device__ __forceinline__ void grid_params(double lo, double hi, int bits, double& scale,
                                            double& zero) {
  lo = fmin(lo, 0.0);
  hi = fmax(hi, 0.0);
  if (lo == hi) {
    lo = -1.0;
    hi = 1.0;
  }
  scale = (hi - lo) / (double)((1 << bits) - 1);
  zero = rint(-lo / scale);
}

// per-channel parameters from the whole initial row (natural order)
__global__ void __launch_bounds__(256) gptq_row_params(GptqParams p, double* pc) {
  const int64_t r = blockIdx.x;
  __shared__ double smin[4], smax[4];
  double lo = INFINITY, hi = -INFINITY;
  for (int64_t c = threadIdx.x; c < p.n; c += 256) {
    const double v = (double)p.W[r * p.ldw + c];
    lo = fmin(lo, v);
    hi = fmax(hi, v);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    lo = fmin(lo, __shfl_xor(lo, off, 64));
    hi = fmax(hi, __shfl_xor(hi, off, 64));
  }
  if ((threadIdx.x & 63) == 0) {
    smin[threadIdx.x >> 6] = lo;
    smax[threadIdx.x >> 6] = hi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    lo = fmin(fmin(smin[0], smin[1]), fmin(smin[2], smin[3]));
    hi = fmax(fmax(smax[0], smax[1]), fmax(smax[2], smax[3]));
    double scale, zero;
    grid_params(lo, hi, p.bits, scale, zero);
    pc[2 * r] = scale;
    pc[2 * r + 1] = zero;
    p.scales[r] = (float)scale;
    p.zeros[r] = (float)zero;
  }
}

// Left-looking product of one block: the four waves split K = jb into
// quarters (each a multiple of KB = 32) and walk theirs in batches of 32 k.
// In MFMA step s of a batch, lane (r = lane % 16, g = lane / 16) supplies
// E[row0 + r][kb + 8 g + s] and, for accumulator tile t, R[kb + 8 g + s][jb +
// 8 r + t]: each lane loads 8 contiguous doubles of E and 8 rows of 8
// contiguous floats of R per batch (16-byte loads), and tile t, column r holds
// block column 8 r + t.
constexpr int KB = 32;

struct GqBatch {
  f64x2_t e[4];       // E[arow][kb + 8 g .. + 7]
  f32x4_t r[8][2];    // R[kb + 8 g + s][jb + 8 r .. + 7]
};

__device__ __forceinline__ void gq_load(GqBatch& B, const double* Eb, const float* Rb, int64_t ldr,
                                        int64_t kb) {
  const double* e = Eb + kb;
#pragma unroll
  for (int q = 0; q < 4; ++q) B.e[q] = *reinterpret_cast<const f64x2_t*>(e + 2 * q);
  const float* r = Rb + kb * ldr;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    B.r[s][0] = *reinterpret_cast<const f32x4_t*>(r + s * ldr);
    B.r[s][1] = *reinterpret_cast<const f32x4_t*>(r + s * ldr + 4);
  }
}

// acc[t] += E R over the batch; `live` false turns the batch into a no-op
// (its E operand is zeroed) without a branch around the accumulators
__device__ __forceinline__ void gq_mma(const GqBatch& B, bool live, f64x4_t (&acc)[8]) {
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const double a = live ? B.e[s >> 1][s & 1] : 0.0;
#pragma unroll
    for (int t = 0; t < 8; ++t)
      acc[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, (double)B.r[s][t >> 2][t & 3], acc[t], 0, 0, 0);
  }
}

// An empty register-only asm hides the value from the optimizer, so that an
// address built from it is recomputed at each use instead of being hoisted
// out of the block loop (one live register per column otherwise).
__device__ __forceinline__ int opaque_int(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// State of one lane in the block's column loop: the lane's 8 columns of its
// row (v), the outputs of the columns it owns, and the grid parameters.
struct InBlock {
  double (&v)[8], (&ev)[8], (&wq)[8], (&tv)[8];
  int (&qv)[8];
  double scale, zero, inv_scale;
  f32x4_t r0, r1;   // staged R row of the next column (this lane's 8 entries)
  double id;        // 1 / R_cc of the next column
};

// Columns 8 O .. 8 O + 7 of the block (owned by lane O of each 16-lane row).
template <int O>
__device__ __forceinline__ void in_block_octet(InBlock& st, const GptqParams& p, const float* Rb,
                                               const double* invd, int part_id, bool row_ok,
                                               int64_t grow, int64_t jb, int ncols, int maxq) {
  if (p.group > 0 && ((8 * O) % p.group) == 0) {
    // parameters of the group [8 O, 8 O + group) from the current values
    const int c = 8 * O;
    double lo = INFINITY, hi = -INFINITY;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int cc = 8 * part_id + q;
      const bool in = cc >= c && cc < c + p.group && cc < ncols;
      lo = in ? fmin(lo, st.v[q]) : lo;
      hi = in ? fmax(hi, st.v[q]) : hi;
    }
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) {
      lo = fmin(lo, __shfl_xor(lo, off, 16));
      hi = fmax(hi, __shfl_xor(hi, off, 16));
    }
    grid_params(lo, hi, p.bits, st.scale, st.zero);
    st.inv_scale = 1.0 / st.scale;
    if (part_id == O && row_ok && c < ncols) {
      const int64_t g = (jb + c) / p.group;
      p.scales[grow * p.ngroups + g] = (float)st.scale;
      p.zeros[grow * p.ngroups + g] = (float)st.zero;
    }
  }
  const bool own = part_id == O;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int c = 8 * O + s;
    // this column's staged R row and 1 / R_cc were read one column ahead;
    // read the next column's now
    const f32x4_t r0v = st.r0, r1v = st.r1;
    const double id = st.id;
    if (c + 1 < BLK) {
      const float* Rn = Rb + (c + 1) * RLD + opaque_int(8 * part_id);
      st.r0 = *reinterpret_cast<const f32x4_t*>(Rn);
      st.r1 = *reinterpret_cast<const f32x4_t*>(Rn + 4);
      st.id = invd[opaque_int(c + 1)];
    }
    // owner lane: round column c
    const double t = fma(st.v[s], st.inv_scale, st.zero);
    const double q = fmin(fmax(rint(t), 0.0), (double)maxq);
    const double w_q = st.scale * (q - st.zero);
    const double e = (st.v[s] - w_q) * id;
    // select now (an empty asm pins each result here): left to itself the
    // compiler keeps every octet's candidates live and selects at the end
    st.ev[s] = own ? e : st.ev[s];
    st.wq[s] = own ? w_q : st.wq[s];
    st.tv[s] = own ? t : st.tv[s];
    st.qv[s] = own ? (int)q : st.qv[s];
    asm volatile("" : "+v"(st.ev[s]), "+v"(st.wq[s]), "+v"(st.tv[s]), "+v"(st.qv[s]));
    const double eb = bcast_row<O>(e);
    // compensate the later columns of the block held by this lane (the
    // staged row is zero at and before column c); the next column first
    if (s + 1 < 8) st.v[s + 1] = fma(-eb, (double)(s + 1 < 4 ? r0v[(s + 1) & 3] : r1v[(s + 1) & 3]), st.v[s + 1]);
#pragma unroll
    for (int q2 = 0; q2 < 8; ++q2) {
      if (q2 == s + 1) continue;
      st.v[q2] = fma(-eb, (double)(q2 < 4 ? r0v[q2 & 3] : r1v[q2 & 3]), st.v[q2]);
    }
    // keep the scheduler from hoisting later columns' reads (one straight
    // line of 128 columns would otherwise be scheduled as a whole)
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int... O>
__device__ __forceinline__ void in_block_octets(InBlock& st, const GptqParams& p, const float* Rb,
                                                const double* invd, int part_id, bool row_ok,
                                                int64_t grow, int64_t jb, int ncols, int maxq,
                                                std::integer_sequence<int, O...>) {
  (in_block_octet<O>(st, p, Rb, invd, part_id, row_ok, grow, jb, ncols, maxq), ...);
}

__global__ void __launch_bounds__(GT, 1) gptq_kernel(GptqParams p) {
  extern __shared__ __align__(16) double gl[];
  double* part = gl;                                       // 4 x RT x BLK doubles
  float* Rb = reinterpret_cast<float*>(gl + 4 * RT * BLK);  // BLK x RLD floats
  double* invd = reinterpret_cast<double*>(Rb + BLK * RLD); // BLK doubles

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t row0 = (int64_t)blockIdx.x * RT;
  // in-block mapping
  const int lrow = 4 * wave + (lane >> 4);  // 0..15
  const int part_id = lane & 15;            // 8 columns each
  const int64_t grow = row0 + lrow;
  const bool row_ok = grow < p.m;
  const int maxq = (1 << p.bits) - 1;

  double scale = 1.0, zero = 0.0;
  if (p.group == 0 && row_ok) {
    scale = p.pc[2 * grow];
    zero = p.pc[2 * grow + 1];
  }
  double inv_scale = 1.0 / scale;

  const int nblocks = (int)((p.n + BLK - 1) / BLK);
  for (int b = 0; b < nblocks; ++b) {
    const int64_t jb = (int64_t)b * BLK;
    const int ncols = (int)min<int64_t>(BLK, p.n - jb);

    // ---- 1. left-looking update on the matrix cores ----
    {
      f64x4_t acc[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[t] = f64x4_t{0.0, 0.0, 0.0, 0.0};
      const int64_t kq = jb / 4;  // multiple of KB
      const int64_t k_lo = kq * wave;
      const int nb = (int)(kq / KB);
      if (nb > 0) {
        const int r = lane & 15, g = lane >> 4;
        // rows past m read row m - 1 (results discarded); columns past n in
        // the last block read the next row of R or its padding (rows k < jb
        // <= n - 2, so the reads stay inside R; results discarded)
        const int64_t arow = min<int64_t>(row0 + r, p.m - 1);
        const double* Eb = p.E + arow * p.ldE + 8 * g;
        const float* Rg = p.R + (int64_t)(8 * g) * p.ldr + jb + 8 * r;
        // two register buffers, each refilled a whole batch of MFMAs before
        // it is consumed; the scheduling barriers keep the compiler from
        // sinking the loads next to their use
        GqBatch A, B;
        gq_load(A, Eb, Rg, p.ldr, k_lo);
        for (int i = 0; i < nb; i += 2) {
          gq_load(B, Eb, Rg, p.ldr, k_lo + (int64_t)KB * min(i + 1, nb - 1));
          __builtin_amdgcn_sched_barrier(0);
          gq_mma(A, true, acc);
          __builtin_amdgcn_sched_barrier(0);
          gq_load(A, Eb, Rg, p.ldr, k_lo + (int64_t)KB * min(i + 2, nb - 1));
          __builtin_amdgcn_sched_barrier(0);
          gq_mma(B, i + 1 < nb, acc);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // partial of this wave -> LDS; f64 16x16 accumulator layout: register v
      // holds row 4 v + lane / 16; tile t, lane column r is block column 8 r + t
      double* pw = part + wave * RT * BLK;
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) pw[(4 * v + (lane >> 4)) * BLK + 8 * (lane & 15) + t] = acc[t][v];
    }
    // stage the diagonal block of R: strictly upper part (zeros on and below
    // the diagonal, so compensating with a row needs no column test) and the
    // reciprocal diagonal
    if (ncols == BLK) {
#pragma unroll
      for (int q = 0; q < BLK * BLK / 4 / GT; ++q) {
        const int e4 = tid + GT * q;
        const int i = e4 / (BLK / 4), j = (e4 % (BLK / 4)) * 4;
        f32x4_t v = *reinterpret_cast<const f32x4_t*>(p.R + (jb + i) * p.ldr + jb + j);
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = (j + u > i) ? v[u] : 0.f;
        *reinterpret_cast<f32x4_t*>(Rb + i * RLD + j) = v;
      }
    } else {
      for (int e = tid; e < BLK * BLK; e += GT) {
        const int i = e / BLK, j = e % BLK;
        Rb[i * RLD + j] = (i < ncols && j < ncols && j > i) ? p.R[(jb + i) * p.ldr + jb + j] : 0.f;
      }
    }
    for (int i = tid; i < BLK; i += GT) {
      const int64_t ii = min<int64_t>(jb + i, p.n - 1);
      const double rd = (double)p.R[ii * p.ldr + ii];
      invd[i] = (i < ncols) ? 1.0 / rd : 0.0;
    }
    __syncthreads();
    // reduce the four partials and add W (natural column perm[jb + c]);
    // rows past m and columns past n read clamped addresses and get zero
    for (int e = tid; e < RT * BLK; e += GT) {
      const int r = e / BLK, c = e % BLK;
      const int64_t gr = row0 + r;
      const bool ok = gr < p.m && c < ncols;
      const int64_t wr = min<int64_t>(gr, p.m - 1);
      const int64_t wc = colmap(p, min<int64_t>(jb + c, p.n - 1));
      const double w = (double)p.W[wr * p.ldw + wc];
      const double s4 = part[e] + part[RT * BLK + e] + part[2 * RT * BLK + e] + part[3 * RT * BLK + e];
      part[e] = ok ? w - s4 : 0.0;
    }
    __syncthreads();

    // ---- 2. sequential columns of the block ----
    double v[8], ev[8], wq[8], tv[8];
    int qv[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      v[s] = part[lrow * BLK + 8 * part_id + s];
      ev[s] = 0.0;
      wq[s] = 0.0;
      tv[s] = 0.0;
      qv[s] = 0;
    }
    // Every column of the block is walked (past ncols the values, invd and
    // staged rows are zero and nothing is stored), so the loop has no exit
    // inside and the reads of R and invd do not wait on the chain.  The 16
    // octets of columns are a compile-time sequence, so the owner lane of a
    // column (broadcast by DPP) and the register holding it are constants.
    InBlock st{v, ev, wq, tv, qv, scale, zero, inv_scale,
               *reinterpret_cast<const f32x4_t*>(Rb + 8 * part_id),
               *reinterpret_cast<const f32x4_t*>(Rb + 8 * part_id + 4), invd[0]};
    in_block_octets(st, p, Rb, invd, part_id, row_ok, grow, jb, ncols, maxq,
                    std::make_integer_sequence<int, 16>{});
    scale = st.scale;
    zero = st.zero;
    inv_scale = st.inv_scale;
    // ---- 3. write errors and outputs of this block ----
    if (row_ok) {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int c = 8 * part_id + s;
        if (c < ncols) {
          const int64_t j = jb + c;
          p.E[grow * p.ldE + j] = ev[s];
          const int64_t nc = colmap(p, j);
          p.codes[grow * p.n + nc] = (uint8_t)qv[s];
          if (p.What) p.What[grow * p.n + nc] = (float)wq[s];
          if (p.pre) p.pre[grow * p.n + nc] = (float)tv[s];
        }
      }
    }
    // E of this block is read by the other waves of this workgroup in the
    // next block's product: the barrier's workgroup-scope release/acquire
    // orders those global stores before the loads (the lines of the new
    // columns were never cached by this CU)
    __syncthreads();
  }
}

int64_t lde(int64_t n) { return (n + 15) / 16 * 16; }

}  // namespace

size_t gptq_ws_bytes(int64_t m, int64_t n) {
  return align_up((size_t)m * lde(n) * sizeof(double), 256) +
         align_up((size_t)m * 2 * sizeof(double), 256);
}

kronq_status gptq_launch(const float* W, int64_t m, int64_t n, int64_t ldw, const float* R,
                         int64_t ldr, const int32_t* perm, int bits, int group, uint8_t* codes,
                         float* scales, float* zeros, float* What, float* pre_round, void* ws,
                         size_t ws_bytes, hipStream_t s) {
  (void)ws_bytes;
  if (group > 0 && (BLK % group != 0 || group % 8 != 0))
    return fail(KRONQ_EUNSUPPORTED, "kronq_gptq_quantize: group %d must be a multiple of 8 dividing %d",
                group, BLK);
  GptqParams p{};
  p.W = W;
  p.m = m;
  p.n = n;
  p.ldw = ldw;
  p.R = R;
  p.ldr = ldr;
  p.perm = perm;
  p.bits = bits;
  p.group = group;
  p.ngroups = group > 0 ? (int)(n / group) : 1;
  p.codes = codes;
  p.scales = scales;
  p.zeros = zeros;
  p.What = What;
  p.pre = pre_round;
  p.E = static_cast<double*>(ws);
  p.ldE = lde(n);
  double* pc = reinterpret_cast<double*>(static_cast<char*>(ws) +
                                         align_up((size_t)m * p.ldE * sizeof(double), 256));
  p.pc = pc;
  if (group == 0) {
    hipLaunchKernelGGL(gptq_row_params, dim3((unsigned)m), dim3(256), 0, s, p, pc);
    KQ_LAUNCHED("gptq_row_params");
  }
  const size_t lds = 4 * RT * BLK * sizeof(double) + BLK * RLD * sizeof(float) + BLK * sizeof(double);
  KQ_HIP(hipFuncSetAttribute((const void*)gptq_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)lds));
  hipLaunchKernelGGL(gptq_kernel, dim3((unsigned)((m + RT - 1) / RT)), dim3(GT), lds, s, p);
  KQ_LAUNCHED("gptq_kernel");
  return KRONQ_OK;
}

}  // namespace kronq
