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
constexpr int CT = 256;        // chain threads (waves 0..3)
constexpr int GT = 512;        // threads: chain waves, then four product waves

struct GptqParams {
  const float* W;          // the weights (per-channel grids)
  const float* Wp;         // what the start values begin from: W, or W plus the
                           // drift shift of earlier units (asymmetric correction)
  const float* X2;         // drift shift from earlier columns of a unit (m x n,
                           // processing order), added after the unit's grid; or NULL
  int unit;                // columns of a unit: the group, or 128 per-channel
  int64_t m, n, ldw, ldwp;
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
  double* D64;             // staged images of the diagonal blocks, nblocks x 128 x 128
  bool vec_out;            // natural order, n % 8 == 0, outputs 16-byte aligned
};

// value of `x` held by lane 16 * (lane / 16) + O, for every lane: DPP
// row_newbcast (lane O of each 16-lane row to the whole row), a 64-bit value
// moved as two halves
template <int O>
__device__ __forceinline__ double bcast_row(double x) {
  const long long b = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_mov_dpp((int)b, 0x150 + O, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_mov_dpp((int)(b >> 32), 0x150 + O, 0xf, 0xf, false);
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

// An empty register-only asm hides the value from the optimizer, so that an
// address built from it is recomputed where it is used instead of being
// hoisted out of the block loop (one live register per octet otherwise).
__device__ __forceinline__ int opaque_int(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

constexpr int KB = 32;   // k per batch of the product

// ---------------------------------------------------------------------------
// Main kernel.  One workgroup owns RT = 16 rows; its eight waves have two
// roles that run side by side, one of each on every SIMD:
//   chain waves 0..3   walk the 128 columns of block b one after another
//                      (rows 4 w .. 4 w + 3, 16 lanes per row, 8 columns per
//                      lane), then write the block's outputs and errors;
//   product waves 4..7 meanwhile form block b + 1's start values from the
//                      errors of blocks 0 .. b - 1 (E R on the fp64 matrix
//                      cores) and, once block b's errors are out, add block
//                      b's share.
// LDS (exactly 160 KiB):
//   Rsq  128 x 128 doubles: the diagonal block of R, strictly upper part
//        (zeros on and below the diagonal, so compensating with a row needs no
//        column test); row 127 has no entries above the diagonal and holds
//        1 / R_cc instead
//   P0   16 x 128 doubles: W minus the first half of the K range's product
//   P1   16 x 128 doubles: the second half's product
// The start value of (row, column) is P0 - P1.
constexpr int SQ = BLK * BLK;   // doubles in Rsq
constexpr size_t kGptqLds = (size_t)(SQ + 2 * RT * BLK) * sizeof(double);
static_assert(kGptqLds == 160 * 1024, "LDS layout");

// Quantize one value onto the grid: grid coordinate t, code q, and the scaled
// error e = (v - w_q) / R_cc with w_q = scale (q - zero).  The column loop and
// the output pass call this same function, so their e agree bit for bit.
struct Quant {
  double t, q, e;
};
__device__ __forceinline__ Quant quant(double v, double scale, double zero, double inv_scale,
                                       double maxq, double id) {
#pragma clang fp contract(off)
  Quant r;
  r.t = fma(v, inv_scale, zero);
  r.q = fmin(fmax(rint(r.t), 0.0), maxq);
  r.e = fma(-scale, r.q - zero, v) * id;
  return r;
}

// ---- chain role ----

struct Chain {
  double v[8];               // this lane's 8 columns of its row
  float x2[8];               // drift shift of those columns from earlier columns of their unit
  f64x2_t rc[4];             // staged R row of the current column (this lane's 8 entries)
  double idc;                // 1 / R_cc of the current column
  double scale, zero, inv_scale;     // grid of the current group
  double oscale, ozero, oinv;        // grid of the group holding this lane's columns
};

__device__ __forceinline__ double rc_at(const Chain& st, int q) { return st.rc[q >> 1][q & 1]; }

// Columns 8 O .. 8 O + 7 of the block (owned by lane O of each 16-lane row).
template <bool DRIFT, int O>
__device__ __forceinline__ void chain_octet(Chain& st, const GptqParams& p, const double* Rsq,
                                            int part_id, bool row_ok, int64_t grow, int64_t jb,
                                            int ncols, double maxq) {
  if (p.group > 0 && ((8 * O) % p.group) == 0) {
    // grid of the group [8 O, 8 O + group) from the current values
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
    const bool mine = 8 * part_id >= c && 8 * part_id < c + p.group;
    st.oscale = mine ? st.scale : st.oscale;
    st.ozero = mine ? st.zero : st.ozero;
    st.oinv = mine ? st.inv_scale : st.oinv;
  }
  if (DRIFT && ((8 * O) % p.unit) == 0) {
    // the unit starting at column 8 O has its grid: add the drift shift of
    // its own earlier columns to its values (it does not depend on rounding)
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int cc = 8 * part_id + q;
      if (cc >= 8 * O && cc < 8 * O + p.unit) st.v[q] += (double)st.x2[q];
    }
  }
  // this lane's entries of row 8 O, and the reciprocal diagonal from column
  // 8 O on: one address per octet (kept out of the block loop by the empty
  // asm), the columns' offsets are immediates
  const double* rb = Rsq + 8 * O * BLK + opaque_int(8 * part_id);
  const double* ib = Rsq + (BLK - 1) * BLK + opaque_int(8 * O);
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int c = 8 * O + s;
    // the next column's staged row and 1 / R_cc (row 127 holds no R entries:
    // column 127 compensates nothing)
    f64x2_t rn[4];
    double idn = 0.0;
    if (c + 1 < BLK - 1) {
#pragma unroll
      for (int q = 0; q < 4; ++q) rn[q] = *reinterpret_cast<const f64x2_t*>(rb + (s + 1) * BLK + 2 * q);
    }
    if (c + 1 < BLK) idn = ib[s + 1];
    // the owner lane quantizes column c; its error goes to the whole row
    const Quant z = quant(st.v[s], st.scale, st.zero, st.inv_scale, maxq, st.idc);
    const double eb = bcast_row<O>(z.e);
    if (c + 1 < BLK) {
      // compensate the later columns held by this lane (the staged row is zero
      // at and before column c); the next column first
      const int nx = (s + 1) & 7;
      st.v[nx] = fma(-eb, rc_at(st, nx), st.v[nx]);
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (q != nx) st.v[q] = fma(-eb, rc_at(st, q), st.v[q]);
    }
    if (c + 1 < BLK - 1) {
#pragma unroll
      for (int q = 0; q < 4; ++q) st.rc[q] = rn[q];
    }
    st.idc = idn;
    // keep the scheduler from hoisting later columns' reads (one straight
    // line of 128 columns would otherwise be scheduled as a whole)
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <bool DRIFT, int... O>
__device__ __forceinline__ void chain_octets(Chain& st, const GptqParams& p, const double* Rsq,
                                             int part_id, bool row_ok, int64_t grow, int64_t jb,
                                             int ncols, double maxq, std::integer_sequence<int, O...>) {
  (chain_octet<DRIFT, O>(st, p, Rsq, part_id, row_ok, grow, jb, ncols, maxq), ...);
}

// Stage diagonal block b (its fp64 image, made once per call) into Rsq.
// Threads t = 0 .. CT - 1; a plain copy of 128 KiB.
__device__ __forceinline__ void stage_rsq(const GptqParams& p, double* Rsq, int b, int t) {
  const f64x2_t* src = reinterpret_cast<const f64x2_t*>(p.D64 + (int64_t)b * SQ);
  f64x2_t* dst = reinterpret_cast<f64x2_t*>(Rsq);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    f64x2_t x[SQ / 2 / CT / 2];
#pragma unroll
    for (int q = 0; q < SQ / 2 / CT / 2; ++q) x[q] = src[t + CT * (q + h * SQ / 2 / CT / 2)];
#pragma unroll
    for (int q = 0; q < SQ / 2 / CT / 2; ++q) dst[t + CT * (q + h * SQ / 2 / CT / 2)] = x[q];
  }
}

template <bool DRIFT>
__device__ __forceinline__ void chain_role(const GptqParams& p, double* gl, int tid) {
  double* Rsq = gl;
  const double* P0 = gl + SQ;
  const double* P1 = P0 + RT * BLK;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int64_t row0 = (int64_t)blockIdx.x * RT;
  const int lrow = 4 * wave + (lane >> 4);  // 0..15
  const int part_id = lane & 15;            // 8 columns each
  const int64_t grow = row0 + lrow;
  const bool row_ok = grow < p.m;
  const double maxq = (double)((1 << p.bits) - 1);

  Chain st;
  st.scale = 1.0;
  st.zero = 0.0;
  if (p.group == 0 && row_ok) {
    st.scale = p.pc[2 * grow];
    st.zero = p.pc[2 * grow + 1];
  }
  st.inv_scale = 1.0 / st.scale;
  st.oscale = st.scale;
  st.ozero = st.zero;
  st.oinv = st.inv_scale;

  const int nblocks = (int)((p.n + BLK - 1) / BLK);
  stage_rsq(p, Rsq, 0, tid);
  __syncthreads();
  for (int b = 0; b < nblocks; ++b) {
    const int64_t jb = (int64_t)b * BLK;
    const int ncols = (int)min<int64_t>(BLK, p.n - jb);
    // ---- the columns of block b ----
    {
      const double* p0 = P0 + lrow * BLK + 8 * part_id;
      const double* p1 = P1 + lrow * BLK + 8 * part_id;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f64x2_t a = *reinterpret_cast<const f64x2_t*>(p0 + 2 * q);
        const f64x2_t c = *reinterpret_cast<const f64x2_t*>(p1 + 2 * q);
        st.v[2 * q] = a[0] - c[0];
        st.v[2 * q + 1] = a[1] - c[1];
        st.rc[q] = *reinterpret_cast<const f64x2_t*>(Rsq + 8 * part_id + 2 * q);
      }
      st.idc = Rsq[(BLK - 1) * BLK];
      if constexpr (DRIFT) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int64_t col = jb + 8 * part_id + q;
          st.x2[q] = (row_ok && col < p.n) ? p.X2[grow * p.n + col] : 0.f;
        }
      }
    }
    // Every column of the block is walked (past ncols the values, staged rows
    // and reciprocals are zero and nothing is stored), so the loop has no exit
    // inside and the reads of the staged rows do not wait on the chain.  The 16
    // octets of columns are a compile-time sequence, so the owner lane of a
    // column (broadcast by DPP) and the register holding it are constants.
    chain_octets<DRIFT>(st, p, Rsq, part_id, row_ok, grow, jb, ncols, maxq,
                 std::make_integer_sequence<int, 16>{});
    // ---- outputs of this lane's columns ----
    // A column's value is final once its own step is done (later steps
    // compensate later columns only), so the owner recomputes its outputs
    // from it with the same arithmetic as in the loop.
    if (row_ok) {
      const double* idr = Rsq + (BLK - 1) * BLK + 8 * part_id;
      double ev[8], wq[8], tv[8];
      int qv[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const Quant z = quant(st.v[s], st.oscale, st.ozero, st.oinv, maxq, idr[s]);
        ev[s] = z.e;
        tv[s] = z.t;
        qv[s] = (int)z.q;
        wq[s] = st.oscale * (z.q - st.ozero);
      }
      const int c0 = 8 * part_id;
      const int64_t j0 = jb + c0;
      if (c0 + 8 <= ncols) {
#pragma unroll
        for (int s = 0; s < 8; s += 2)
          *reinterpret_cast<f64x2_t*>(p.E + grow * p.ldE + j0 + s) = f64x2_t{ev[s], ev[s + 1]};
      } else {
        for (int s = 0; s < 8; ++s)
          if (c0 + s < ncols) p.E[grow * p.ldE + j0 + s] = ev[s];
      }
      if (p.vec_out && c0 + 8 <= ncols) {
        // natural order, 8 consecutive columns, aligned
        const int64_t o = grow * p.n + j0;
        uint32_t c4[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
          c4[h] = (uint32_t)qv[4 * h] | ((uint32_t)qv[4 * h + 1] << 8) | ((uint32_t)qv[4 * h + 2] << 16) |
                  ((uint32_t)qv[4 * h + 3] << 24);
        *reinterpret_cast<uint2*>(p.codes + o) = make_uint2(c4[0], c4[1]);
        if (p.What) {
          *reinterpret_cast<f32x4_t*>(p.What + o) = f32x4_t{(float)wq[0], (float)wq[1], (float)wq[2], (float)wq[3]};
          *reinterpret_cast<f32x4_t*>(p.What + o + 4) = f32x4_t{(float)wq[4], (float)wq[5], (float)wq[6], (float)wq[7]};
        }
        if (p.pre) {
          *reinterpret_cast<f32x4_t*>(p.pre + o) = f32x4_t{(float)tv[0], (float)tv[1], (float)tv[2], (float)tv[3]};
          *reinterpret_cast<f32x4_t*>(p.pre + o + 4) = f32x4_t{(float)tv[4], (float)tv[5], (float)tv[6], (float)tv[7]};
        }
      } else {
        for (int s = 0; s < 8; ++s) {
          if (c0 + s < ncols) {
            const int64_t nc = colmap(p, j0 + s);
            p.codes[grow * p.n + nc] = (uint8_t)qv[s];
            if (p.What) p.What[grow * p.n + nc] = (float)wq[s];
            if (p.pre) p.pre[grow * p.n + nc] = (float)tv[s];
          }
        }
      }
    }
    // The E stores reach the product waves' loads through this barrier's
    // workgroup-scope release/acquire (the lines of a block's columns are
    // never read before they are written, so no stale copy sits in this CU's
    // cache).
    __syncthreads();
    if (b + 1 < nblocks) stage_rsq(p, Rsq, b + 1, tid);
    __syncthreads();
  }
}

// ---- product role ----
//
// Product wave pw = 0..3 covers columns 64 ch .. 64 ch + 63 of the next block
// (ch = pw & 1; four 16 x 16 tiles) over half kh = pw >> 1 of the K range, in
// batches of 32 k.  In MFMA step s of a batch, lane (r = lane % 16, g = lane /
// 16) supplies E[row r][kb + 8 g + s] and, for tile t, R[kb + 8 g + s][64 ch +
// 4 r + t]: each lane loads 8 contiguous doubles of E and 8 rows of 4
// contiguous doubles of R per batch (16-byte loads).  Tile t's lane column r
// is block column 64 ch + 4 r + t; accumulator register v holds row 4 v + g.
// R is read as stored (fp32, exact in fp64) and widened in registers: half the
// bytes of an fp64 copy on the loop's largest stream (down_proj's loop at
// n = 28672 took 168 ms reading an fp64 copy, 126 ms this way).
struct PBatch {
  f64x2_t e[4];      // E[arow][kb + 8 g .. + 7]
  f32x4_t r[8];      // R[kb + 8 g + s][64 ch + 4 r .. + 3]
};

__device__ __forceinline__ void pb_load(PBatch& B, const double* Eg, const float* Rg, int64_t ldr,
                                        int64_t kb) {
  const double* e = Eg + kb;
#pragma unroll
  for (int q = 0; q < 4; ++q) B.e[q] = *reinterpret_cast<const f64x2_t*>(e + 2 * q);
  const float* r = Rg + kb * ldr;
#pragma unroll
  for (int s = 0; s < 8; ++s) B.r[s] = *reinterpret_cast<const f32x4_t*>(r + s * ldr);
}

// The batch's 32 R values are widened first, into registers of their own, and
// only then fed to the matrix cores.  Widened one at a time beside its MFMA,
// each value went to the one register that the MFMA issued just before was
// still reading, and every widening waited for that MFMA: about 28 cycles lost
// per 64-cycle MFMA (down_proj's loop at n = 28672: 129 ms this way against
// 117 ms widened first, codes identical).
__device__ __forceinline__ void pb_mma(const PBatch& B, f64x4_t (&acc)[4]) {
  double cv[8][4];
#pragma unroll
  for (int s = 0; s < 8; ++s)
#pragma unroll
    for (int t = 0; t < 4; ++t) cv[s][t] = (double)B.r[s][t];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const double a = B.e[s >> 1][s & 1];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      acc[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, cv[s][t], acc[t], 0, 0, 0);
  }
}

// fp64 images of R's diagonal blocks, made once per call: each block as staged
// for the column loop, its strictly upper part with zeros on and below the
// diagonal and past n, and in row 127 the reciprocal diagonal.  One workgroup
// per row of the padded block grid.
__global__ void __launch_bounds__(256) gptq_diag64(GptqParams p) {
  const int64_t k = blockIdx.x;
  const int i = (int)(k % BLK);
  const int64_t jb = k - i;
  const int ncols = (int)min<int64_t>(BLK, p.n - jb);
  double* drow = p.D64 + (jb / BLK) * SQ + (int64_t)i * BLK;
  if (i == BLK - 1) {
    for (int j = threadIdx.x; j < BLK; j += 256)
      drow[j] = j < ncols ? 1.0 / (double)p.R[(jb + j) * p.ldr + jb + j] : 0.0;
  } else {
    for (int j = threadIdx.x; j < BLK; j += 256)
      drow[j] = (j > i && j < ncols) ? (double)p.R[k * p.ldr + jb + j] : 0.0;
  }
}

template <bool DRIFT>
__device__ __forceinline__ void product_role(const GptqParams& p, double* gl, int tid) {
  double* P0 = gl + SQ;
  double* P1 = P0 + RT * BLK;
  // wave-uniform: the K and column offsets below are scalar arithmetic
  const int pw = __builtin_amdgcn_readfirstlane(tid >> 6) - CT / 64, lane = tid & 63;
  const int kh = pw >> 1, ch = pw & 1;
  const int r = lane & 15, g = lane >> 4;
  const int64_t row0 = (int64_t)blockIdx.x * RT;
  // rows past m read row m - 1 (results discarded); columns past n in the
  // last block read the start of the next row of the fp64 copy (rows k < jn
  // <= n - 1 when the next block is not empty, so the reads stay inside it;
  // the values are not written there and the results are discarded)
  const int64_t arow = min<int64_t>(row0 + r, p.m - 1);
  const double* Eg = p.E + arow * p.ldE + 8 * g;
  const int nblocks = (int)((p.n + BLK - 1) / BLK);
  double* P = kh == 0 ? P0 : P1;

  // W of the block at column jn for this lane's outputs (first K half only)
  auto load_w = [&](int64_t jn, float (&w)[4][4]) {
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int64_t wr = min<int64_t>(row0 + 4 * v + g, p.m - 1);
        const int64_t wc = colmap(p, min<int64_t>(jn + 64 * ch + 4 * r + t, p.n - 1));
        w[v][t] = DRIFT ? p.Wp[wr * p.ldwp + wc] : p.W[wr * p.ldw + wc];
      }
  };
  // start values of the block at column jn: W - acc (first half), acc (second)
  auto store = [&](int64_t jn, const f64x4_t (&acc)[4], const float (&w)[4][4]) {
    const int ncn = (int)min<int64_t>(BLK, p.n - jn);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = 4 * v + g;
      const bool rok = row0 + row < p.m;
      double o[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int col = 64 * ch + 4 * r + t;
        const double x = kh == 0 ? (double)w[v][t] - acc[t][v] : acc[t][v];
        o[t] = (rok && col < ncn) ? x : 0.0;
      }
      double* d = P + row * BLK + 64 * ch + 4 * r;
      *reinterpret_cast<f64x2_t*>(d) = f64x2_t{o[0], o[1]};
      *reinterpret_cast<f64x2_t*>(d + 2) = f64x2_t{o[2], o[3]};
    }
  };

  {
    // block 0: no product yet
    float w[4][4];
    if (kh == 0) load_w(0, w);
    f64x4_t acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = f64x4_t{0.0, 0.0, 0.0, 0.0};
    store(0, acc, w);
  }
  __syncthreads();
  for (int b = 0; b < nblocks; ++b) {
    const int64_t jb = (int64_t)b * BLK, jn = jb + BLK;
    const bool more = b + 1 < nblocks;
    const float* Rg = p.R + (int64_t)(8 * g) * p.ldr + jn + 64 * ch + 4 * r;
    const int64_t ldrr = p.ldr;
    f64x4_t acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = f64x4_t{0.0, 0.0, 0.0, 0.0};
    float w[4][4];
    if (more && kh == 0) load_w(jn, w);
    // errors of blocks 0 .. b - 1: this half of [0, jb) is 2 b batches
    const int nbat = more ? 2 * b : 0;
    if (nbat > 0) {
      const int64_t k0 = (int64_t)kh * (jb / 2);
      // two register buffers, each refilled a whole batch of MFMAs before it
      // is consumed; the scheduling barriers keep the compiler from sinking
      // the loads next to their use
      PBatch A, B;
      pb_load(A, Eg, Rg, ldrr, k0);
      for (int i = 0; i < nbat; i += 2) {
        pb_load(B, Eg, Rg, ldrr, k0 + (int64_t)KB * (i + 1));
        __builtin_amdgcn_sched_barrier(0);
        pb_mma(A, acc);
        __builtin_amdgcn_sched_barrier(0);
        pb_load(A, Eg, Rg, ldrr, k0 + (int64_t)KB * min(i + 2, nbat - 1));
        __builtin_amdgcn_sched_barrier(0);
        pb_mma(B, acc);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();
    if (more) {
      // block b's errors: this half of [jb, jb + 128)
      PBatch A, B;
      pb_load(A, Eg, Rg, ldrr, jb + BLK / 2 * kh);
      pb_load(B, Eg, Rg, ldrr, jb + BLK / 2 * kh + KB);
      pb_mma(A, acc);
      pb_mma(B, acc);
      store(jn, acc, w);
    }
    __syncthreads();
  }
}

// DRIFT: the asymmetric correction's drift shifts (start values from Wp, X2
// added at unit starts); a separate instantiation so that the plain loop keeps
// its registers
template <bool DRIFT>
__global__ void __launch_bounds__(GT, 1) gptq_kernel(GptqParams p) {
  extern __shared__ __align__(16) double gl[];
  const int tid = threadIdx.x;
  // the role is uniform per wave: a scalar branch; both roles pass the same
  // sequence of barriers
  if (__builtin_amdgcn_readfirstlane(tid >> 6) < CT / 64)
    chain_role<DRIFT>(p, gl, tid);
  else
    product_role<DRIFT>(p, gl, tid);
}

int64_t lde(int64_t n) { return (n + 15) / 16 * 16; }

// row_loss[r] = sum_j E[r][j]^2 over the row's n scaled errors, fp64: one wave
// per row, lanes striding the row, butterfly reduction across the wave.
__global__ void __launch_bounds__(256) gptq_row_loss(const double* E, int64_t ldE, int64_t m,
                                                      int64_t n, double* out) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= m) return;
  const double* e = E + r * ldE;
  double acc = 0.0;
  for (int64_t j = lane; j < n; j += 64) acc = fma(e[j], e[j], acc);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (lane == 0) out[r] = acc;
}

bool aligned(const void* q, size_t a) { return (reinterpret_cast<uintptr_t>(q) % a) == 0; }

}  // namespace

size_t gptq_ws_bytes(int64_t m, int64_t n) {
  return align_up((size_t)m * lde(n) * sizeof(double), 256) +
         align_up((size_t)m * 2 * sizeof(double), 256) +

         (size_t)((n + BLK - 1) / BLK) * SQ * sizeof(double);
}

kronq_status gptq_launch(const float* W, int64_t m, int64_t n, int64_t ldw, const float* R,
                         int64_t ldr, const int32_t* perm, int bits, int group, uint8_t* codes,
                         float* scales, float* zeros, float* What, float* pre_round,
                         double* row_loss, void* ws, size_t ws_bytes, hipStream_t s,
                         const float* Wp, const float* X2) {
  (void)ws_bytes;
  if (group > 0 && (BLK % group != 0 || group % 8 != 0))
    return fail(KRONQ_EUNSUPPORTED, "kronq_gptq_quantize: group %d must be a multiple of 8 dividing %d",
                group, BLK);
  GptqParams p{};
  p.W = W;
  p.Wp = Wp ? Wp : W;
  p.X2 = X2;
  p.unit = group > 0 ? group : BLK;
  p.m = m;
  p.n = n;
  p.ldw = ldw;
  p.ldwp = Wp ? n : ldw;
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
  p.D64 = reinterpret_cast<double*>(reinterpret_cast<char*>(pc) + align_up((size_t)m * 2 * sizeof(double), 256));
  p.vec_out = perm == nullptr && n % 8 == 0 && aligned(codes, 8) && (What == nullptr || aligned(What, 16)) &&
              (pre_round == nullptr || aligned(pre_round, 16));
  if (group == 0) {
    hipLaunchKernelGGL(gptq_row_params, dim3((unsigned)m), dim3(256), 0, s, p, pc);
    KQ_LAUNCHED("gptq_row_params");
  }
  hipLaunchKernelGGL(gptq_diag64, dim3((unsigned)((n + BLK - 1) / BLK * BLK)), dim3(256), 0, s, p);
  KQ_LAUNCHED("gptq_diag64");
  const size_t lds = kGptqLds;
  if (X2) {
    KQ_HIP(hipFuncSetAttribute((const void*)gptq_kernel<true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)lds));
    hipLaunchKernelGGL(gptq_kernel<true>, dim3((unsigned)((m + RT - 1) / RT)), dim3(GT), lds, s, p);
  } else {
    KQ_HIP(hipFuncSetAttribute((const void*)gptq_kernel<false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)lds));
    hipLaunchKernelGGL(gptq_kernel<false>, dim3((unsigned)((m + RT - 1) / RT)), dim3(GT), lds, s, p);
  }
  KQ_LAUNCHED("gptq_kernel");
  if (row_loss) {
    hipLaunchKernelGGL(gptq_row_loss, dim3((unsigned)((m + 3) / 4)), dim3(256), 0, s,
                       (const double*)p.E, p.ldE, m, n, row_loss);
    KQ_LAUNCHED("gptq_row_loss");
  }
  return KRONQ_OK;
}

}  // namespace kronq
