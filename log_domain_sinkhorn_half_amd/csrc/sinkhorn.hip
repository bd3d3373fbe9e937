// Log-domain Sinkhorn half-steps for squared-Euclidean cost on MI355X (gfx950).
//
// Method: page "FlashSinkhorn: Trasporto Ottimo Entropico Consapevole delle I/O su GPU", section
// "Metodologia".  Part "1. Riformulazione in Forma di Attenzione" (Proposizione 1) rewrites the
// stabilised update
//   f_i <- -eps LSE_j[(g_j - C_ij)/eps + log b_j],  C_ij = ||x_i - y_j||^2
// as f_i = ||x_i||^2 - eps * LSE_j[(2 x_i.y_j + beta_j)/eps] with the per-column
// bias beta_j = g_j - ||y_j||^2 + eps log b_j: a dot-product score matrix with a
// bias, reduced by a row log-sum-exp.  Part "2. Kernel di Streaming e Tassellazione"
// streams it: query tiles stay on chip (row-stationary), key tiles stream past
// them, the LSE is accumulated online and the n x m scores never reach HBM.  The g update is the same
// kernel with the clouds exchanged.
//
// MI355X design (not the pages' Triton/A100 design):
//  * Scores come from v_mfma_f32_16x16x32_bf16.  On gfx950 fp32 MFMA shares
//    issue with the VALU, while bf16 MFMA overlaps partly with the exp/add
//    stream that bounds small-d problems.  Scores are produced directly in
//    base-2 units, lambda = log2(e)/eps, so the VALU does only exp2 + add.
//  * The bf16 MFMA sums each group of 8 products (one lane group) exactly and
//    adds the group sums to the fp32 accumulator with round-to-nearest.  The
//    fp32 path uses that: every coordinate of x and of v = 2*lambda*y is split
//    into a "grid" part (a multiple of a power-of-two quantum, at most 8 bits)
//    plus two bf16 remainder parts.  Grid products, the grid part of the bias
//    lambda*beta_j and the running row offset -m_i are all multiples of one
//    quantum Q, so their sum is exact in fp32 in any order; they occupy the
//    first K slots.  The seven remainder products per coordinate (and the bias
//    remainder) are small and come after, so the only rounding happens at the
//    magnitude of the final exponent.  Scores are then accurate far below the
//    fp32 rounding of the output potential.
//  * bf16 inputs: raw bf16 values (products are exact in fp32); the half bias
//    beta_j/2 goes in through the accumulator and one FMA per element applies
//    the 2*lambda scale and the offset.
//  * Online LSE with a lazy offset: a workgroup sets its row offsets from the
//    first key tile's maximum plus a headroom, and moves them only when a
//    chunk's partial sums exceed 2^112 (rare), so the hot loop has no max or
//    rescale.  Such a chunk is recomputed with its exact maximum; offsets are
//    integers, so rescaling is an exact power of two.
//  * Key chunks are staged through LDS (double buffered) and shared by the
//    four (or eight) waves of a workgroup; each wave keeps its own query tiles
//    in VGPRs.
//  * Key ranges are split across workgroups when rows alone cannot fill the
//    256 CUs; the partial (max, sum) pairs are merged by a small kernel.
//  * Norms, log-weights, the bias and the final potential are formed in fp64.
//
// Beyond the half-step (same page, section "Metodologia", part "3. Differenziazione e
// Ottimizzazione del Secondo Ordine"; and the section "Significato e Affermazioni" on costs):
//  * transport application: barycentric projection and gradient in one P.V
//    pass over the score tiles with lazy row offsets, and the plan applied to
//    any matrix with offsets fixed by the potentials (k_bary);
//  * Hessian-vector products of the OT value, from plan products only
//    (conjugate gradients on a Schur system, then an assembly; the quadratic
//    term in one pass whose weights carry the direction's dot products);
//  * the cosine cost, as the squared-Euclidean cost between normalised points.

#include <hip/hip_runtime.h>

#include <float.h>
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <type_traits>
#include <utility>

#include "sinkhorn.h"

// Built-in workspace of sinkhorn_solve_noalloc: SK_NOALLOC_MAX_BYTES of device
// memory per GPU the library runs on, held until the process ends.  Host code
// never uses this name as a device address: it takes each device's address
// from hipGetSymbolAddress (scratch_address below).
static __device__ __align__(256) unsigned char scratch[SK_NOALLOC_MAX_BYTES];

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

#define SK_HD __host__ __device__

namespace {

#include "host_layout.h"


thread_local char g_err[512] = "";

void set_err(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

// ---------------------------------------------------------------------------
// bf16 helpers (round to nearest even on the bit pattern)
// ---------------------------------------------------------------------------
__device__ __forceinline__ u16 bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (u16)(u >> 16);
}
__device__ __forceinline__ float bf16_f(u16 h) { return __uint_as_float(((uint32_t)h) << 16); }
__device__ __forceinline__ u16 bf16_of(double v) { return bf16_rne((float)v); }

constexpr u16 BF16_ONE = 0x3F80;

// Eight bf16 values as one 16-byte vector (element 0 in the low half of x).
__device__ __forceinline__ u4 pack8(const u16 (&v)[8]) {
  return u4{(uint32_t)v[0] | ((uint32_t)v[1] << 16), (uint32_t)v[2] | ((uint32_t)v[3] << 16),
            (uint32_t)v[4] | ((uint32_t)v[5] << 16), (uint32_t)v[6] | ((uint32_t)v[7] << 16)};
}

// Exponent k of the smallest power of two q = 2^k with |v| / q <= 255 (k = 0
// when v == 0).  Callers form q and 1/q exactly with ldexp.
__device__ __forceinline__ int grid_exponent(double vmax) {
  if (!(vmax > 0.0)) return 0;
  int e;
  const double mant = frexp(vmax / 255.0, &e);  // vmax/255 = mant * 2^e, mant in [0.5, 1)
  return mant == 0.5 ? e - 1 : e;
}

// Grid part and two bf16 remainder parts of v: v ~ g + r1 + r2 with g a
// multiple of q, |v - g| <= q/2 and a residual below 2^-18 q.  inv_q = 1/q
// exactly (q is a power of two).
struct Parts {
  u16 g, r1, r2;
};
__device__ __forceinline__ Parts grid_split(double v, double q, double inv_q) {
  const double g = rint(v * inv_q) * q;
  double r = v - g;
  Parts p;
  p.g = bf16_of(g);
  p.r1 = bf16_of(r);
  r -= (double)bf16_f(p.r1);
  p.r2 = bf16_of(r);
  return p;
}

// s * 2^(m_old - m_new) for integer offsets m_old <= m_new.  Done with ldexp, not
// exp2: v_exp_f32 flushes results below 2^-126 to zero, which would drop a large
// partial sum whenever the offset jumps by more than 126.
__device__ __forceinline__ float rescale(float s, float m_old, float m_new) {
  const float d = m_old - m_new;
  return d < -300.f ? 0.f : ldexpf(s, (int)d);
}

// Coordinate k of a point cloud stored as fp32 or bf16.
__device__ __forceinline__ float coord(const void* P, size_t k, int in_bf16) {
  return in_bf16 ? bf16_f(static_cast<const u16*>(P)[k]) : static_cast<const float*>(P)[k];
}

// ---------------------------------------------------------------------------
// Set-up kernels
// ---------------------------------------------------------------------------
// Centring.  The squared-Euclidean cost only depends on differences x_i - y_j,
// so both clouds of a problem are moved by one common vector c (the centre of
// their joint bounding box) before anything else is formed: the potentials do
// not change, while the norms and the dot-product scores shrink from the size
// of |x| to the size of the clouds' spread.  The cosine cost is not
// translation-invariant and keeps c = 0.
//
// Order-preserving unsigned code of a float, so that atomicMin / atomicMax on
// codes give the minimum / maximum of the values in any order (deterministic).
__device__ __forceinline__ unsigned ordered_code(float v) {
  const unsigned u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ordered_value(unsigned c) {
  return __uint_as_float((c & 0x80000000u) ? (c & 0x7FFFFFFFu) : ~c);
}

// Per (problem, side, coordinate) bounding box of the clouds: box[(b*2+side)*2d + t]
// is the code of the minimum of coordinate t, box[... + d + t] of the maximum.
// The slots start at 0xFFFFFFFF (minima) and 0 (maxima).  grid: (point chunks,
// 2 sides, batch).  For d <= 256 the 256 threads of a block hold 256/d points side
// by side (thread = point * d + coordinate, so a load instruction reads whole
// rows); wider points take one coordinate per thread and loop over the rest.
// Minima and maxima meet in LDS, then once per block and coordinate in memory.
__global__ __launch_bounds__(256) void k_bbox(const void* __restrict__ X, const void* __restrict__ Y, int in_bf16,
                                              int n, int m, int d, unsigned* __restrict__ box) {
  __shared__ unsigned lmin[SK_MAX_D], lmax[SK_MAX_D];
  const int side = blockIdx.y, b = blockIdx.z;
  const int rows = side == 0 ? n : m;
  const void* P = side == 0 ? X : Y;
  const int tid = threadIdx.x;
  for (int k = tid; k < d; k += 256) {
    lmin[k] = 0xFFFFFFFFu;
    lmax[k] = 0u;
  }
  __syncthreads();
  const int per = d <= 256 ? 256 / d : 1;  // points per pass of the block
  const int lanes = d <= 256 ? per * d : 256;
  if (tid < lanes) {
    const int pp = d <= 256 ? tid / d : 0;
    for (int t = d <= 256 ? tid % d : tid; t < d; t += 256) {
      float lo = INFINITY, hi = -INFINITY;
      for (long long i = (long long)blockIdx.x * per + pp; i < rows; i += (long long)gridDim.x * per) {
        const float v = coord(P, ((size_t)b * rows + i) * d + t, in_bf16);
        lo = fminf(lo, v);
        hi = fmaxf(hi, v);
      }
      atomicMin(&lmin[t], ordered_code(lo));
      atomicMax(&lmax[t], ordered_code(hi));
      if (d <= 256) break;
    }
  }
  __syncthreads();
  unsigned* bx = box + (size_t)(b * 2 + side) * 2 * d;
  for (int k = tid; k < d; k += 256) {
    atomicMin(&bx[k], lmin[k]);
    atomicMax(&bx[d + k], lmax[k]);
  }
}

// Centre c of each problem (fp64 [batch][d]) from the two boxes, and the largest
// |coordinate - c| of each side (maxabs[side*batch + b], rounded up to a float;
// it sizes the grid quantum of the split operand layout).  bf16 inputs take a
// bf16 centre, so that x - c can be exact in bf16, and only when the joint box
// leaves out the origin in some coordinate (otherwise the norms shrink little);
// an uncentred bf16 problem gets inexact[b] = 2, so no exactness check runs.
// One workgroup per problem.
__global__ __launch_bounds__(256) void k_centre(const unsigned* __restrict__ box, int d, int batch, int in_bf16,
                                                int centre, double* __restrict__ cen, float* __restrict__ maxabs,
                                                unsigned* __restrict__ inexact) {
  __shared__ double red[2][256];
  __shared__ int off_origin;
  const int b = blockIdx.x;
  const unsigned* bx = box + (size_t)b * 4 * d;  // side 0: [0, 2d), side 1: [2d, 4d)
  if (threadIdx.x == 0) off_origin = 0;
  __syncthreads();
  if (in_bf16)
    for (int t = threadIdx.x; t < d; t += 256) {
      const double lo = fmin((double)ordered_value(bx[t]), (double)ordered_value(bx[2 * d + t]));
      const double hi = fmax((double)ordered_value(bx[d + t]), (double)ordered_value(bx[3 * d + t]));
      if (lo > 0.0 || hi < 0.0) off_origin = 1;
    }
  __syncthreads();
  if (in_bf16 && centre && !off_origin) {
    centre = 0;
    if (threadIdx.x == 0) inexact[b] = 2u;
  }
  double mx0 = 0.0, mx1 = 0.0;
  for (int t = threadIdx.x; t < d; t += 256) {
    const double lo0 = ordered_value(bx[t]), hi0 = ordered_value(bx[d + t]);
    const double lo1 = ordered_value(bx[2 * d + t]), hi1 = ordered_value(bx[3 * d + t]);
    double c = 0.0;
    if (centre) {
      c = 0.5 * (fmin(lo0, lo1) + fmax(hi0, hi1));  // exact: a sum of two floats, halved
      if (!isfinite(c)) c = 0.0;
      if (in_bf16) c = (double)bf16_f(bf16_rne((float)c));
    }
    cen[(size_t)b * d + t] = c;
    mx0 = fmax(mx0, fmax(fabs(hi0 - c), fabs(lo0 - c)));
    mx1 = fmax(mx1, fmax(fabs(hi1 - c), fabs(lo1 - c)));
  }
  red[0][threadIdx.x] = mx0;
  red[1][threadIdx.x] = mx1;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      red[0][threadIdx.x] = fmax(red[0][threadIdx.x], red[0][threadIdx.x + w]);
      red[1][threadIdx.x] = fmax(red[1][threadIdx.x], red[1][threadIdx.x + w]);
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    maxabs[b] = __double2float_ru(red[0][0]);
    maxabs[batch + b] = __double2float_ru(red[1][0]);
  }
}

// bf16 inputs keep their values in the operands, so a problem is centred only if
// every x - c of both clouds is a bf16 value itself (true for clouds far from the
// origin compared with their spread, where centring matters).  Sets inexact[b]
// otherwise (one atomic per block).  Problems already left uncentred are
// skipped.  grid: (element chunks, batch, 2 sides).
__global__ __launch_bounds__(256) void k_bf16_exact(const u16* __restrict__ X, const u16* __restrict__ Y,
                                                    long long nx, long long ny, int d,
                                                    const double* __restrict__ cen, unsigned* __restrict__ inexact) {
  __shared__ int any_bad;
  const int b = blockIdx.y, side = blockIdx.z;
  if (inexact[b] != 0u) return;  // uniform across the block
  if (threadIdx.x == 0) any_bad = 0;
  __syncthreads();
  const long long cnt = side == 0 ? nx : ny;
  const u16* P = (side == 0 ? X : Y) + (size_t)b * cnt;
  bool bad = false;
  const double* cb_ = cen + (size_t)b * d;
  for (long long k = (long long)blockIdx.x * 256 + threadIdx.x; k < cnt; k += (long long)gridDim.x * 256) {
    const int t = cnt < (1LL << 31) ? (int)((unsigned)k % (unsigned)d) : (int)(k % d);
    const double v = (double)bf16_f(P[k]) - cb_[t];
    bad |= (double)bf16_f(bf16_rne((float)v)) != v;
  }
  if (bad) any_bad = 1;
  __syncthreads();
  if (threadIdx.x == 0 && any_bad) atomicOr(&inexact[b], 1u);
}

// Problems whose differences are not all bf16 values keep c = 0.
__global__ __launch_bounds__(256) void k_cen_fix(const unsigned* __restrict__ inexact, int d, double* __restrict__ cen) {
  const int b = blockIdx.x;
  if (inexact[b] == 0u) return;
  for (int t = threadIdx.x; t < d; t += 256) cen[(size_t)b * d + t] = 0.0;
}

// Coordinate t of point r (row index over all problems) of a cloud, minus the centre.
__device__ __forceinline__ double ccoord(const void* P, size_t r, int t, int d, int in_bf16,
                                         const double* __restrict__ cen, int b) {
  return (double)coord(P, r * d + t, in_bf16) - cen[(size_t)b * d + t];
}

// Norms (fp64), log-weights (fp64) and inverse norms of one cloud, from the
// centred points x - c (under the cosine cost: the normalised points, not
// centred).  One thread per point.  bf16 inputs: the norm of the centred bf16
// values (x - c is a bf16 value there).
template <int MODE>
__global__ __launch_bounds__(256) void k_init_rows(const void* __restrict__ P, const float* __restrict__ w, int rows,
                                                   int d, int in_bf16, int cosine, const double* __restrict__ cen,
                                                   double* __restrict__ norm, double* __restrict__ logw,
                                                   double* __restrict__ rnorm) {
  const int b = blockIdx.y;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows) return;
  const size_t r = (size_t)b * rows + i;
  const double* cb_ = cen + (size_t)b * d;
  double rn = 1.0;
  if (MODE == MODE_SPLIT && cosine) {
    double raw = 0.0;
    for (int t = 0; t < d; ++t) {
      const double v = coord(P, r * d + t, in_bf16);
      raw += v * v;
    }
    rn = raw > 0.0 ? 1.0 / sqrt(raw) : 0.0;  // a zero point stays zero
  }
  double nrm = 0.0;
  for (int t = 0; t < d; ++t) {
    double v = (double)coord(P, r * d + t, in_bf16) * rn - cb_[t];
    if (MODE == MODE_BF16) v = (double)bf16_f(bf16_of(v));
    nrm += v * v;
  }
  norm[r] = nrm;
  rnorm[r] = rn;
  logw[r] = log((double)w[r]);
}

// Operand rows of one cloud (queries of its half-steps), one thread per 16-byte
// segment (8 K slots) of a row; rows past the points are zero.
//   split layout (fp32 inputs up to SK_MAX_D_SPLIT, and the cosine cost): the
//     query side of the K-slot layout above, from x*rn - c;
//   hi/lo layout (wider fp32 inputs): (x_h, x_h, x_l) per coordinate, x = x_h + x_l
//     the centred coordinate in two bf16 parts (paired with the key's v_h, v_l, v_h);
//   bf16 inputs: the centred bf16 values, zero-padded.
// Needs rnorm from k_init_rows.
template <int MODE>
__global__ __launch_bounds__(256) void k_init_ops(const void* __restrict__ P, int rows, int rows_pad, int d, int KP,
                                                  int in_bf16, const float* __restrict__ maxabs,
                                                  const double* __restrict__ cen, const double* __restrict__ rnorm,
                                                  u16* __restrict__ opnd) {
  const int b = blockIdx.y;
  const int vpr = KP / 8;
  const long long gtid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gtid >= (long long)rows_pad * vpr) return;
  const int i = (int)(gtid / vpr), k0 = (int)(gtid % vpr) * 8;
  u16* dst = opnd + ((size_t)b * rows_pad + i) * KP + k0;
  if (i >= rows) {
    *reinterpret_cast<u4*>(dst) = u4{0, 0, 0, 0};
    return;
  }
  const size_t r = (size_t)b * rows + i;
  const double* cb_ = cen + (size_t)b * d;
  const double rn = rnorm[r];
  auto val = [&](int t) { return (double)coord(P, r * d + t, in_bf16) * rn - cb_[t]; };
  u16 v[8];
  if (MODE == MODE_BF16) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (k0 + e < d) ? bf16_of(val(k0 + e)) : (u16)0;
  } else if (MODE == MODE_HILO) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = k0 + e, t = k / 3;
      u16 h = 0;
      if (t < d) {
        const double x = val(t);
        const u16 xh = bf16_of(x);
        h = (k % 3 == 2) ? bf16_of(x - (double)bf16_f(xh)) : xh;
      }
      v[e] = h;
    }
  } else {
    const int qe = grid_exponent(maxabs[b]);
    const double q = ldexp(1.0, qe), iq = ldexp(1.0, -qe);
    const int cb = split_corr_begin(d);
    if (k0 < cb) {
      // grid section: offset slots (zero here, set in registers), ones, grid parts
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k = k0 + e;
        v[e] = (k >= 2 && k <= 4) ? BF16_ONE : ((k >= 5 && k < 5 + d) ? grid_split(val(k - 5), q, iq).g : (u16)0);
      }
    } else {
      // corrections (x_g x_g x_1 x_2 x_1 x_1 x_2 per coordinate), then the two ones
      // of the bias remainder; a segment touches at most two coordinates
      const int t0 = (k0 - cb) / 7;
      const Parts zero{0, 0, 0};
      const Parts p0 = t0 < d ? grid_split(val(t0), q, iq) : zero;
      const Parts p1 = t0 + 1 < d ? grid_split(val(t0 + 1), q, iq) : zero;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int rel = k0 + e - cb;
        u16 v_ = 0;
        if (rel < 7 * d) {
          const bool first = rel / 7 == t0;
          const int sl = rel % 7;
          const u16 pg = first ? p0.g : p1.g, pr1 = first ? p0.r1 : p1.r1, pr2 = first ? p0.r2 : p1.r2;
          v_ = (sl <= 1) ? pg : ((sl == 3 || sl == 6) ? pr2 : pr1);
        } else if (rel == 7 * d || rel == 7 * d + 1) {
          v_ = BF16_ONE;
        }
        v[e] = v_;
      }
    }
  }
  *reinterpret_cast<u4*>(dst) = pack8(v);
}

// Grid and remainder parts of v = l2*yc (l2 = 2*lambda, yc the centred or
// normalised coordinate, exact in fp64) for the key operand: v is formed in fp64
// and carried as vh + vl (two floats), so the remainder takes one fp32 rounding,
// as in the fp64 split.  q = 2^k and iq = 1/q must be normal floats.
__device__ __forceinline__ Parts key_split(double yc, float l2, float q, float iq) {
  const double v = (double)l2 * yc;
  const float vh = (float)v;
  const float vl = (float)(v - (double)vh);
  const float g = rintf(vh * iq) * q;
  const float r = (vh - g) + vl;  // vh - g is exact: both are multiples of ulp(vh)
  Parts p;
  p.g = bf16_rne(g);
  p.r1 = bf16_rne(r);
  p.r2 = bf16_rne(r - bf16_f(p.r1));
  return p;
}

// Bias lambda*(pot - norm + eps*logw) of one key in parts: bp[0..2] its multiple
// of the grid quantum Q (exact in three bf16 parts), bp[3..4] the remainder.
// Keys of zero weight and padding keys (real == false) take NEG_BIG alone.
__device__ __forceinline__ void bias_parts(bool real, float pot, double norm, double logw, float lam, float eps,
                                           double Q, double iQ, u16 (&bp)[5]) {
  double bias = (double)NEG_BIG;
  if (real) {
    bias = (double)lam * ((double)pot - norm + (double)eps * logw);
    if (!(bias >= (double)NEG_BIG)) bias = (double)NEG_BIG;  // zero weight (-inf) or underflow
  }
  for (int e = 0; e < 5; ++e) bp[e] = 0;
  if (bias <= (double)NEG_BIG) {
    bp[0] = bf16_of(bias);
  } else {
    const double bg = rint(bias * iQ) * Q;
    bp[0] = bf16_of(bg);
    bp[1] = bf16_of(bg - (double)bf16_f(bp[0]));
    bp[2] = bf16_of(bg - (double)bf16_f(bp[0]) - (double)bf16_f(bp[1]));
    const double br = bias - bg;
    bp[3] = bf16_of(br);
    bp[4] = bf16_of(br - (double)bf16_f(bp[3]));
  }
}

// Key operand rows for one half-step (fp32 inputs): v = 2*lambda*y and the bias
// lambda*(pot - norm + eps*logw) in grid + remainder parts; writes the grid
// quantum Q = q_query * q_key of each problem to qgrid.  Work items are 16-byte
// segments of a row, consecutive across the threads of a stride, so the stores
// are coalesced.
//
// The coordinate parts depend only on the cloud and lambda.  *tag holds the bit
// pattern of the lambda they were last built for (0: none).  When it equals
// lam, only the five bias slots of each row are rewritten (one key per thread);
// otherwise every segment is, and the tag is cleared.  Only the half-step kernel that follows on
// the stream sets the tag, after every segment of this launch has been written;
// a clear written during this launch cannot change any thread's decision, since
// neither the old tag nor 0 equals lam.
__global__ __launch_bounds__(256) void k_prep_keys(const void* __restrict__ P, int in_bf16,
                                                   const double* __restrict__ rnorm, const double* __restrict__ cen,
                                                   const float* __restrict__ pot,
                                                   const double* __restrict__ norm, const double* __restrict__ logw,
                                                   int keys, int keys_pad, int d, int KP, float lam, float eps,
                                                   const float* __restrict__ qmax, const float* __restrict__ kmax,
                                                   float* __restrict__ qgrid, unsigned* __restrict__ tag,
                                                   u16* __restrict__ kb) {
  const int b = blockIdx.y;
  const int vpr = KP / 8;
  const int cb = split_corr_begin(d);
  const int sb1 = (cb + 7 * d) / 8, sb2 = (cb + 7 * d + 1) / 8;  // segments of the remainder slots
  const bool fresh = *tag == __float_as_uint(lam);
  // the grid is sized for a full rebuild; a bias-only pass needs one thread per key
  if (fresh && (long long)blockIdx.x * blockDim.x >= keys_pad) return;
  const long long gtid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long stride = (long long)gridDim.x * blockDim.x;
  if (!fresh && gtid == 0 && b == 0) *tag = 0u;
  const double lam2 = 2.0 * (double)lam;
  const int qqe = grid_exponent(qmax[b]);
  const int qke = grid_exponent(lam2 * (double)kmax[b]);
  const double qk = ldexp(1.0, qke), iqk = ldexp(1.0, -qke);
  const double Q = ldexp(1.0, qqe + qke), iQ = ldexp(1.0, -(qqe + qke));
  if (gtid == 0) qgrid[b] = (float)Q;
  // fp32 coordinate splits unless the key quantum leaves the normal float range
  const bool f32 = qke > -100 && qke < 100;
  const float l2f = 2.f * lam, qkf = ldexpf(1.f, qke), iqkf = ldexpf(1.f, -qke);
  if (fresh) {
    for (long long j = gtid; j < keys_pad; j += stride) {
      u16 bp[5];
      const size_t r = (size_t)b * keys + (j < keys ? j : 0);
      bias_parts(j < keys, pot[r], norm[r], logw[r], lam, eps, Q, iQ, bp);
      u16* row = kb + ((size_t)b * keys_pad + j) * KP;
      row[2] = bp[0];
      row[3] = bp[1];
      row[4] = bp[2];
      row[cb + 7 * d] = bp[3];
      row[cb + 7 * d + 1] = bp[4];
    }
    return;
  }
  const long long nwork = (long long)keys_pad * vpr;
  for (long long wi = gtid; wi < nwork; wi += stride) {
    const int j = (int)(wi / vpr), seg = (int)(wi % vpr);
    const int k0 = seg * 8;
    const bool real = j < keys;
    const size_t r = (size_t)b * keys + j;
    const double rn = real ? rnorm[r] : 1.0;
    auto split = [&](int t) {
      const double yc = (double)coord(P, r * d + t, in_bf16) * rn - cen[(size_t)b * d + t];
      return f32 ? key_split(yc, l2f, qkf, iqkf) : grid_split(lam2 * yc, qk, iqk);
    };
    u16 bp[5] = {0, 0, 0, 0, 0};
    if (seg == 0 || seg == sb1 || seg == sb2) {
      const size_t rr = real ? r : (size_t)b * keys;
      bias_parts(real, pot[rr], norm[rr], logw[rr], lam, eps, Q, iQ, bp);
    }
    u16 v[8];
    if (k0 < cb) {
      // grid section: offset slots (ones), bias grid parts, coordinate grid parts;
      // segment 0 holds slots 0..7, so its bias slots have fixed positions
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k = k0 + e;
        u16 val = 0;
        if (seg == 0 && e <= 1)
          val = BF16_ONE;
        else if (seg == 0 && e <= 4)
          val = bp[e - 2];
        else if (k < 5 + d && real)
          val = split(k - 5).g;
        v[e] = val;
      }
    } else {
      // corrections (key side v_1 v_2 v_g v_g v_1 v_2 v_1 per coordinate), then the
      // bias remainder; a segment touches at most two coordinates
      const int t0 = (k0 - cb) / 7;
      const Parts zero{0, 0, 0};
      const Parts p0 = (real && t0 < d) ? split(t0) : zero;
      const Parts p1 = (real && t0 + 1 < d) ? split(t0 + 1) : zero;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int rel = k0 + e - cb;
        u16 val = 0;
        if (rel < 7 * d) {
          const bool first = rel / 7 == t0;  // selects values: a reference select would go to scratch
          const u16 pg = first ? p0.g : p1.g, p1r = first ? p0.r1 : p1.r1, p2r = first ? p0.r2 : p1.r2;
          const int sl = rel % 7;
          val = (sl == 2 || sl == 3) ? pg : ((sl == 1 || sl == 5) ? p2r : p1r);
        } else if (rel == 7 * d) {
          val = bp[3];
        } else if (rel == 7 * d + 1) {
          val = bp[4];
        }
        v[e] = val;
      }
    }
    *reinterpret_cast<u4*>(kb + ((size_t)b * keys_pad + j) * KP + k0) =
        u4{(uint32_t)v[0] | ((uint32_t)v[1] << 16), (uint32_t)v[2] | ((uint32_t)v[3] << 16),
           (uint32_t)v[4] | ((uint32_t)v[5] << 16), (uint32_t)v[6] | ((uint32_t)v[7] << 16)};
  }
}

// Fill n floats with v.
__global__ __launch_bounds__(256) void k_fill_f32(float* __restrict__ p, int n, float v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// Zero-fill n 16-byte words (used instead of a memset so callers may capture it).
__global__ __launch_bounds__(256) void k_zero(u4* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = u4{0, 0, 0, 0};
}

// Copy of the status word to a caller's device word.
__global__ void k_copy_u32(const unsigned* __restrict__ src, unsigned* __restrict__ dst) {
  if (threadIdx.x == 0) *dst = *src;
}

// Start values of the set-up words: bounding-box slots (minima 0xFFFFFFFF, maxima
// 0, see k_bbox), the bf16 centring flags, the status word and the four lambda tags.
__global__ __launch_bounds__(256) void k_init_words(unsigned* __restrict__ box, int d, int batch,
                                                    unsigned* __restrict__ inexact, unsigned* __restrict__ status,
                                                    unsigned* __restrict__ tags) {
  const long long n = 4LL * batch * d;
  const long long i0 = (long long)blockIdx.x * blockDim.x + threadIdx.x, st = (long long)gridDim.x * blockDim.x;
  for (long long i = i0; i < n; i += st) box[i] = ((i / d) % 2 == 0) ? 0xFFFFFFFFu : 0u;
  for (long long i = i0; i < batch; i += st) inexact[i] = 0u;
  if (i0 == 0) {
    status[0] = 0u;
    for (int k = 0; k < 4; ++k) tags[k] = 0u;
  }
}

// Bias vector scale * (pot - norm + eps*logw) per key: scale 1/2 (bf16 inputs:
// the MFMA's product is x.y, scaled by 2 lambda afterwards) or lambda (hi/lo
// operands: the product is already 2 lambda x.y); padding -> -1e30.
__global__ __launch_bounds__(256) void k_prep_bias(const float* __restrict__ pot, const double* __restrict__ norm,
                                                   const double* __restrict__ logw, int keys, int keys_pad,
                                                   float eps, float scale, float* __restrict__ hb) {
  const int b = blockIdx.y;
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= keys_pad) return;
  float v = NEG_BIG;
  if (j < keys) {
    const size_t r = (size_t)b * keys + j;
    v = (float)((double)scale * ((double)pot[r] - norm[r] + (double)eps * logw[r]));
    if (!(v >= NEG_BIG)) v = NEG_BIG;
  }
  hb[(size_t)b * keys_pad + j] = v;
}

// ---------------------------------------------------------------------------
// The streaming half-step kernel
// ---------------------------------------------------------------------------
typedef float f16v __attribute__((ext_vector_type(16)));

__device__ __forceinline__ bf16x8 as_bf16x8(u4 v) { return __builtin_bit_cast(bf16x8, v); }
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// MFMA tile shapes.  A = key operand (rows = keys), B = query operand (columns =
// queries), D[key][query].  Every lane holds 8 consecutive K slots of one key
// (A) or one query (B): lane = col + MW * grp holds slots [8*grp, 8*grp+8) of the
// instruction's KI slots for row/column `col`.  Output element `o` of a lane is
// D[key_of(o, grp)][col].
template <int MW>
struct Tile;
template <>
struct Tile<16> {  // v_mfma_f32_16x16x32_bf16
  static constexpr int KI = 32, NOUT = 4;
  using Acc = f4;
  static __device__ __forceinline__ Acc mma(u4 a, u4 b, Acc c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ int key_of(int o, int grp) { return 4 * grp + o; }
};
template <>
struct Tile<32> {  // v_mfma_f32_32x32x16_bf16
  static constexpr int KI = 16, NOUT = 16;
  using Acc = f16v;
  static __device__ __forceinline__ Acc mma(u4 a, u4 b, Acc c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ int key_of(int o, int grp) { return 8 * (o / 4) + 4 * grp + (o % 4); }
};

// Offset slots (query side, instruction 0, lane group 0, elements 0..1) <- -m as two bf16 parts.
__device__ __forceinline__ void set_offset(u4& q, float off, bool owner) {
  if (!(off <= 1e30f)) off = 1e30f;
  if (!(off >= -1e30f)) off = -1e30f;
  const u16 h = bf16_rne(off);
  const u16 l = bf16_rne(off - bf16_f(h));
  if (owner) q.x = (uint32_t)h | ((uint32_t)l << 16);
}

// New offset from a chunk maximum: an integer that two bf16 parts hold exactly
// and, on the fp32 path, a multiple of the grid quantum Q.  Two bf16 parts hold
// 16 significant bits, so past 2^21 the quantum grows; once it exceeds the
// headroom the exponents are no longer safe from overflow and flush, and
// `coarse` is set (scores beyond the supported range of 2^22 base-2 units).
__device__ __forceinline__ float offset_from_max(float mx, float Q, bool& coarse) {
  float mq = floorf(mx);
  if (!(fabsf(mq) < 1e30f)) return mq;
  float quantum = fmaxf(Q, 1.f);
  if (fabsf(mq) >= 65536.f) quantum = fmaxf(quantum, ldexpf(1.f, ilogbf(mq) - 15));
  coarse |= quantum > HEADROOM;
  return floorf(mq / quantum) * quantum;
}

// Bits of the status word in the workspace (an OR over every launch since the
// last init): the header's SK_FLAG_SCORE_RANGE and SK_FLAG_NONFINITE.
constexpr unsigned FLAG_SCORE_RANGE = 1u, FLAG_NONFINITE = 2u;
__device__ __forceinline__ void flag_if(unsigned* status, bool cond, unsigned bit) {
  if (cond && status != nullptr) atomicOr(status, bit);
}

// Launch shape per (path, K chunks of 32 slots): tile width MW, query tiles per
// wave R, key tiles per LDS chunk TC.  Wide 32x32 tiles halve the MFMA count per
// score for small K; large K keeps 16x16 tiles so the query operand fits in VGPRs.
// For 12..19 chunks two query tiles per wave and two key tiles per chunk halve
// the LDS operand reads per score while two workgroups still fit a CU's LDS.
// 9..11 chunks (d = 28..43) take 32x32 tiles with one query tile per wave
// (about 220 VGPRs; measured 4% faster than 16x16 tiles at d = 32).
__host__ __device__ constexpr bool cfg_wide_k(int mode, int nch) { return mode == MODE_SPLIT && nch >= 12 && nch <= 19; }
// bf16 operands wider than 256 slots (d > 256) switch to 16x16 tiles with one
// query tile per wave: the query operand alone then takes up to 128 VGPRs.
__host__ __device__ constexpr int cfg_MW(int mode, int nch) {
  return mode == MODE_BF16 ? (nch <= 8 ? 32 : 16) : ((nch <= 2 || (nch >= 9 && nch <= 11)) ? 32 : 16);
}
__host__ __device__ constexpr int cfg_R(int mode, int nch) {
  return cfg_MW(mode, nch) == 32 ? (nch == 1 ? (mode == MODE_SPLIT ? 3 : 4) : (nch <= 4 ? 2 : 1))
                                 : (nch <= 4 ? 4 : (nch <= 8 ? 2 : (cfg_wide_k(mode, nch) ? 2 : 1)));
}
__host__ __device__ constexpr int cfg_TC(int mode, int nch) {
  // bf16 d = 65..256 (8-wave workgroups): 4 key tiles per chunk, measured +5% at d = 128
  return (mode == MODE_SPLIT && nch == 1) ? 8
         : (mode == MODE_BF16 && nch >= 3 && nch <= 8)
             ? 4
             : (cfg_MW(mode, nch) == 32 ? (nch <= 2 ? 2 : 1) : (cfg_wide_k(mode, nch) ? 2 : 1));
}
__host__ __device__ constexpr int cfg_waves(int mode, int nch) {
  return (mode == MODE_SPLIT && nch == 1) ? 3 : ((mode == MODE_BF16 && nch > 20) ? 1 : 2);
}

// Waves per workgroup.  Every wave scores its own query tiles against the key
// chunk the workgroup stages in LDS, so more waves per workgroup divide the key
// operand's global and LDS-store traffic per query.  Measured with 8 waves:
// +10% at d = 64 (fp32), +2% at d = 128 (bf16), -8% for 64 problems at d = 32.
__host__ __device__ constexpr int cfg_NW(int mode, int nch) {
  return ((mode == MODE_SPLIT && nch >= 12 && nch <= 19) || (mode == MODE_BF16 && nch >= 3 && nch <= 8)) ? 8 : 4;
}

// Compile-time parity of a chunk within a workgroup's range: selects the LDS
// buffer and the register set of the prefetch.
template <int P>
struct Par {
  static constexpr int value = P;
};

// Workgroups go to the accelerator's XCDs round-robin in dispatch order (x
// fastest), and each XCD has its own L2.  For batched problems this remaps
// dispatch slots so that every XCD runs one contiguous range of logical blocks:
// the row blocks of one problem then share an L2 (measured +3% on 64 problems of
// 2048 points; single problems lose 1-2%, so they keep the plain order).
struct Blk {
  int x, y, z;
};
__device__ __forceinline__ Blk xcd_block() {
  const int gx = gridDim.x, gy = gridDim.y, n = gx * gy * gridDim.z;
  if (gridDim.z == 1) return {(int)blockIdx.x, (int)blockIdx.y, 0};
  const int p = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
  const int q = n / NXCD, r = n % NXCD, xcd = p % NXCD, k = p / NXCD;
  const int l = (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + k;
  return {l % gx, (l / gx) % gy, l / (gx * gy)};
}

// The next half-step's key bias, written where a potential is finalised (the
// fused update of the page's part "2. Kernel di Streaming e Tassellazione": score,
// bias, reduction and potential in one pass).  The rows of this half-step are
// the keys of the next one, so once p_i is known its bias there follows:
// lambda'(p_i - |x_i|^2 + eps' log w_i) in grid parts into the five bias slots of
// row i of the split key operand (fp32 path; only valid while that operand's
// coordinate parts are built for lambda'), or (p_i - |x_i|^2 + eps' log w_i)/2
// into the half-bias vector (bf16 path).  The values are the ones the
// preparation kernels would write, so skipping them changes no result.
struct NextBias {
  u16* kb;              // split key operand of the next half-step (fp32 path), or nullptr
  float* hb;            // bias vector of the next half-step (bf16 and hi/lo paths), or nullptr
  const double* logw;   // log-weights of this half-step's rows
  const float* qmax;    // largest |coordinate| of the next half-step's query cloud, per problem
  const float* kmax;    // the same for this half-step's rows (the next keys)
  float lam, eps;       // the next half-step's lambda and eps
  float hscale;         // scale of the bias vector: 1/2 (bf16 path) or lambda (hi/lo path)
  int rows_pad, KP, cb, d;
};

__device__ __forceinline__ void write_next_bias(const NextBias& nb, int b, int q, float pot, double norm,
                                                double logw) {
  if (nb.kb != nullptr) {
    const int qqe = grid_exponent(nb.qmax[b]);
    const int qke = grid_exponent(2.0 * (double)nb.lam * (double)nb.kmax[b]);
    const double Q = ldexp(1.0, qqe + qke), iQ = ldexp(1.0, -(qqe + qke));
    u16 bp[5];
    bias_parts(true, pot, norm, logw, nb.lam, nb.eps, Q, iQ, bp);
    u16* row = nb.kb + ((size_t)b * nb.rows_pad + q) * nb.KP;
    row[2] = bp[0];
    row[3] = bp[1];
    row[4] = bp[2];
    row[nb.cb + 7 * nb.d] = bp[3];
    row[nb.cb + 7 * nb.d + 1] = bp[4];
  } else if (nb.hb != nullptr) {
    float v = (float)((double)nb.hscale * ((double)pot - norm + (double)nb.eps * logw));
    if (!(v >= NEG_BIG)) v = NEG_BIG;
    nb.hb[(size_t)b * nb.rows_pad + q] = v;
  }
}

// The plan applied to one vector, sum_j P_ij w_j (page "FlashSinkhorn: Trasporto
// Ottimo Entropico Consapevole delle I/O su GPU", section "Metodologia", part
// "3. Differenziazione e Ottimizzazione del Secondo Ordine": the streaming HVP
// is a sequence of such vector-transport products, one per conjugate-gradient
// step of the Hessian solve here), through the half-step kernel: the offsets are fixed by the rows'
// half-step values T_i (M_i = lambda (|x_i|^2 - T_i), so the weights 2^(s - M_i)
// sum to about 1) and the kernel sums w_j 2^(s - M_i) beside 2^(s - M_i), one
// fp32 FMA per score; the split partials (W, S) go to k_wv_merge.
struct WvArgs {
  const float* w;    // the vector, [batch][keys] fp32
  const float* lse;  // the rows' half-step values T_i, [batch][rows]
};

// TCX overrides the key tiles per chunk (0: cfg_TC) and RX the query tiles per
// wave (0: cfg_R), for small problems.  WV: the one-vector plan product above
// instead of the half-step, 1 with the weight sums, 2 without them (the sums
// depend on the potentials and offsets only, so repeated products with the same
// potentials reuse those of their first pass).
template <int MODE, int NCH, int TCX = 0, int WV = 0, int RX = 0>
__global__ __launch_bounds__(64 * cfg_NW(MODE, NCH)) __attribute__((amdgpu_waves_per_eu(cfg_waves(MODE, NCH)))) void k_lse(
    const u16* __restrict__ Q, const u16* __restrict__ K, const float* __restrict__ hb,
    const float* __restrict__ qgrid, const double* __restrict__ qnorm, float* __restrict__ out,
    float2* __restrict__ part, int rows, int rows_pad, int keys, int keys_pad, int chunks_per_split, int batch,
    float lam2, double inv_lam, unsigned* __restrict__ tag, unsigned tag_val, unsigned* __restrict__ status,
    NextBias nb, WvArgs wv) {
  constexpr int MW = cfg_MW(MODE, NCH), R = RX ? RX : cfg_R(MODE, NCH), TC = TCX ? TCX : cfg_TC(MODE, NCH);
  using T = Tile<MW>;
  using Acc = typename T::Acc;
  constexpr int KP = NCH * 32;
  constexpr int NI = KP / T::KI;   // MFMA instructions per tile
  constexpr int NO = T::NOUT;      // outputs per lane per tile
  constexpr int LROW = KP + (MW == 16 ? 16 : 8);  // LDS row stride (elements); the pad avoids bank conflicts
  constexpr int CK = TC * MW;      // keys per chunk
  constexpr int VPR = KP / 8;      // 16-byte vectors per key row
  constexpr int NVEC = CK * VPR;
  constexpr int NW = cfg_NW(MODE, NCH), NT = 64 * NW;  // waves, threads per workgroup
  constexpr int NLD = (NVEC + NT - 1) / NT;
  constexpr int QPW = R * MW;      // queries per wave
  // fp32 split layout with 9..11 K chunks (32x32 tiles, one query tile per
  // wave, MFMA-bound): exact per-tile maxima move the offsets without ever
  // recomputing a chunk (see `step`).  Measured at d = 32, n = m = 16384: 16%
  // faster for unit-variance clouds (whose score spread makes the lazy offsets
  // redo chunks), 3% slower for clouds scaled by 1/sqrt(d); the batch of 64
  // problems of 2048 points +23%.  For 2..8 chunks (16x16 tiles, up to four
  // query tiles) the per-tile maxima cost 10-50%, and 12..19 chunks have no
  // registers to spare.
  constexpr bool EXACT = !WV && MODE == MODE_SPLIT && NCH >= 9 && NCH <= 11;
  static_assert(!WV || CK <= NT, "one vector element per thread and chunk");
  // the last workgroup's query rows may run past the padded rows into the slack rows
  static_assert(NW * QPW - gcd_c(NW * QPW, ROW_PAD) <= SLACK, "query over-read beyond the slack rows");
  static_assert(CK % 4 == 0 && CK / 4 <= NT, "one 4-key bias vector per thread");
  // chunks must tile the padded key range: keys past it (slack rows) are not prepared
  static_assert(ROW_PAD % CK == 0 && CK <= SLACK, "a key chunk must divide the row padding");
  // One spare row per buffer takes the stores of threads past the end of a chunk.
  __shared__ __attribute__((aligned(16))) u16 lds[2][(CK + 1) * LROW];
  __shared__ __attribute__((aligned(16))) float ldsb[2][CK];
  __shared__ __attribute__((aligned(16))) float ldsw[WV ? 2 : 1][WV ? CK : 4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane / MW, col = lane % MW;
  const Blk blk = xcd_block();
  const int b = blk.z;
  const int qbase = blk.x * (NW * QPW) + wave * QPW;
  // The key operand's preparation (the previous launch on the stream) is
  // complete: record the lambda its coordinate parts now hold.
  if (tag != nullptr && tid == 0 && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0) *tag = tag_val;
  const u16* Qb = Q + (size_t)b * rows_pad * KP;
  const u16* Kb = K + (size_t)b * keys_pad * KP;
  const float* hbb = (MODE == MODE_BF16) ? hb + (size_t)b * keys_pad : nullptr;
  const float qg = (MODE == MODE_SPLIT) ? qgrid[b] : 1.f;

  u4 bq[R][NI];
#pragma unroll
  for (int c = 0; c < R; ++c)
#pragma unroll
    for (int i = 0; i < NI; ++i)
      bq[c][i] = *reinterpret_cast<const u4*>(Qb + (size_t)(qbase + MW * c + col) * KP + i * T::KI + grp * 8);

  const int total_chunks = (keys + CK - 1) / CK;
  const int c0 = blk.y * chunks_per_split;
  const int c1 = min(total_chunks, c0 + chunks_per_split);

  float m[R], s[R];
#pragma unroll
  for (int c = 0; c < R; ++c) {
    m[c] = EXACT ? 0.f : -FLT_MAX;  // EXACT: the offset slots start at zero
    s[c] = 0.f;
  }
  if (EXACT) {
#pragma unroll
    for (int c = 0; c < R; ++c) set_offset(bq[c][0], 0.f, grp == 0);
  }
  // WV: fixed offsets.  On the fp32 path the query operand carries the grid
  // multiple mo of M_i and the rest, sub (below the grid quantum), scales the
  // row's two sums alike, so it is subtracted on the VALU only where it could
  // overflow them (fine).  On the bf16 path m = M_i enters the exponent's FMA.
  float ws[R], sub[R];
  bool fine = false;
  if constexpr (WV) {
    bool coarse = false;
#pragma unroll
    for (int c = 0; c < R; ++c) {
      ws[c] = 0.f;
      sub[c] = 0.f;
      const int q = qbase + MW * c + col;
      double M = 0.0;
      if (q < rows) {
        const size_t r = (size_t)b * rows + q;
        M = (qnorm[r] - (double)wv.lse[r]) / inv_lam;
      }
      if (!(fabs(M) < 1e30)) M = 0.0;
      if (MODE == MODE_SPLIT) {
        const float mo = offset_from_max((float)M, qg, coarse);
        set_offset(bq[c][0], -mo, grp == 0);
        sub[c] = (float)(M - (double)mo);
        fine |= !(sub[c] <= 32.f);
      } else {
        m[c] = (float)M;
      }
    }
    flag_if(status, coarse && lane == 0, FLAG_SCORE_RANGE);
    fine = __any(fine);
  }

  u4 pre[2][NLD];
  f4 preb[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  float prew[2] = {0.f, 0.f};
  // Loads past the end of a chunk land in the slack rows that follow every
  // operand buffer, so they need no guard; their LDS stores go to a spare row.
  auto gload = [&](int chunk, auto par) {
    constexpr int P = decltype(par)::value;
    const u16* src = Kb + (size_t)chunk * CK * KP;
#pragma unroll
    for (int i = 0; i < NLD; ++i) pre[P][i] = *reinterpret_cast<const u4*>(src + (size_t)(tid + NT * i) * 8);
    if (MODE == MODE_BF16) preb[P] = *reinterpret_cast<const f4*>(hbb + (size_t)chunk * CK + (tid % (CK / 4)) * 4);
    if (WV) {
      const int j = chunk * CK + tid;  // keys past the end (zero weight) take 0
      prew[P] = (tid < CK && j < keys) ? wv.w[(size_t)b * keys + j] : 0.f;
    }
  };
  auto lstore = [&](auto par) {
    constexpr int P = decltype(par)::value;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int v = min(tid + NT * i, NVEC);  // NVEC maps to the spare row
      *reinterpret_cast<u4*>(&lds[P][(v / VPR) * LROW + (v % VPR) * 8]) = pre[P][i];
    }
    if (MODE == MODE_BF16 && tid < CK / 4) *reinterpret_cast<f4*>(&ldsb[P][tid * 4]) = preb[P];
    if (WV && tid < CK) ldsw[WV ? P : 0][tid] = prew[P];
  };
  // Scores of key tile t of the chunk in buffer buf against the R query tiles.
  auto tile = [&](int buf, int t, Acc (&acc)[R]) {
    Acc cinit;
#pragma unroll
    for (int o = 0; o < NO; ++o) cinit[o] = 0.f;
    if (MODE == MODE_BF16) {
#pragma unroll
      for (int o = 0; o < NO; o += 4) {
        const f4 v = *reinterpret_cast<const f4*>(&ldsb[buf][t * MW + T::key_of(o, grp)]);
        cinit[o] = v[0];
        cinit[o + 1] = v[1];
        cinit[o + 2] = v[2];
        cinit[o + 3] = v[3];
      }
    }
#pragma unroll
    for (int c = 0; c < R; ++c) acc[c] = cinit;
    // bf16 operands: a wave issuing its MFMA chain takes priority over the
    // exp/add stream of the other waves on its SIMD (measured +1% to +2% at
    // d = 128; alternating the two streams between wave groups with barriers,
    // and interleaving the next tile's MFMAs into this tile's exps, were slower)
    if (MODE == MODE_BF16) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const u4 ka = *reinterpret_cast<const u4*>(&lds[buf][(t * MW + col) * LROW + i * T::KI + grp * 8]);
#pragma unroll
      for (int c = 0; c < R; ++c) acc[c] = T::mma(ka, bq[c][i], acc[c]);
    }
    if (MODE == MODE_BF16) __builtin_amdgcn_s_setprio(0);
  };
  // Base-2 exponent of a score relative to the current offset.
  auto expo = [&](float v, int c) -> float {
    if (MODE == MODE_BF16) return fmaf(v, lam2, -m[c]);
    return v;
  };
  auto raw = [&](float v) -> float {
    if (MODE == MODE_BF16) return v * lam2;
    return v;
  };
  // s += sum of exp2 over a lane's outputs: NO exps and NO adds (pairwise tree).
  auto accumulate = [&](const Acc (&acc)[R]) {
#pragma unroll
    for (int c = 0; c < R; ++c) {
      float e[NO];
#pragma unroll
      for (int o = 0; o < NO; ++o) e[o] = __builtin_amdgcn_exp2f(expo(acc[c][o], c));
#pragma unroll
      for (int w = 1; w < NO; w *= 2)
#pragma unroll
        for (int o = 0; o + w < NO; o += 2 * w) e[o] += e[o + w];
      s[c] += e[0];
    }
  };
  // WV: s += sum of the weights and ws += sum of weight x vector element over
  // a lane's outputs of key tile t (its vector elements from LDS, four keys per
  // 16-byte read).
  auto accumulate_w = [&](const Acc (&acc)[R], int buf, int t, auto fine_c) {
    constexpr bool FINE = decltype(fine_c)::value;
    float wl[NO];
#pragma unroll
    for (int o = 0; o < NO; o += 4) {
      const f4 v = *reinterpret_cast<const f4*>(&ldsw[WV ? buf : 0][t * MW + T::key_of(o, grp)]);
      wl[o] = v[0];
      wl[o + 1] = v[1];
      wl[o + 2] = v[2];
      wl[o + 3] = v[3];
    }
#pragma unroll
    for (int c = 0; c < R; ++c) {
      float e[NO];
#pragma unroll
      for (int o = 0; o < NO; ++o) e[o] = __builtin_amdgcn_exp2f(FINE ? acc[c][o] - sub[c] : expo(acc[c][o], c));
      float w0 = 0.f, w1 = 0.f;
#pragma unroll
      for (int o = 0; o < NO; o += 2) {
        w0 = fmaf(e[o], wl[o], w0);
        w1 = fmaf(e[o + 1], wl[o + 1], w1);
      }
      ws[c] += w0 + w1;
      if constexpr (WV == 1) {
#pragma unroll
        for (int w = 1; w < NO; w *= 2)
#pragma unroll
          for (int o = 0; o + w < NO; o += 2 * w) e[o] += e[o + w];
        s[c] += e[0];
      }
    }
  };
  // combine a value over the lanes that hold the same query
  auto lanes_max = [&](float v) {
#pragma unroll
    for (int w = MW; w < 64; w *= 2) v = fmaxf(v, __shfl_xor(v, w));
    return v;
  };
  auto lanes_sum = [&](float v) {
#pragma unroll
    for (int w = MW; w < 64; w *= 2) v += __shfl_xor(v, w);
    return v;
  };

  // One chunk: score the keys in LDS buffer P (chunk ci, P = parity of ci - c0),
  // load chunk ci+1 and move it from registers into
  // buffer P^1.  Register set Q holds the chunk that buffer Q takes next.
  auto step = [&](int ci, auto par) {
    constexpr int P = decltype(par)::value;
    const int buf = P;
    // Chunk ci+1 goes to register set P^1 (an unconditional, clamped load keeps
    // the wait before its LDS store exact).  Keeping two chunks in flight was
    // measured 5-10% slower on the MFMA-heavy shapes and 2% on d <= 3.
    gload(min(ci + 1, c1 - 1), Par<P ^ 1>{});

    if constexpr (WV) {
      if constexpr (MODE == MODE_SPLIT && NCH == 1 && TC == 8) {
        // d <= 3: unrolled as in the half-step (one tile's MFMAs overlap the
        // previous tile's exps), with the rare fine offsets as a separate copy
        auto tiles = [&](auto fine_c) {
#pragma unroll
          for (int t = 0; t < TC; ++t) {
            Acc acc[R];
            tile(buf, t, acc);
            accumulate_w(acc, buf, t, fine_c);
          }
        };
        if (fine)
          tiles(std::true_type{});
        else
          tiles(std::false_type{});
      } else {
#pragma unroll 1
        for (int t = 0; t < TC; ++t) {
          Acc acc[R];
          tile(buf, t, acc);
          if (fine)
            accumulate_w(acc, buf, t, std::true_type{});
          else
            accumulate_w(acc, buf, t, std::false_type{});
        }
      }
      if (ci + 1 < c1) lstore(Par<P ^ 1>{});
      __syncthreads();
      return;
    }

    if constexpr (EXACT) {
      // Each tile's scores come out of the MFMA relative to the current offsets.
      // The first tile of the range sets them (its maximum + HEADROOM); later, a
      // query whose tile maximum passes its offset by more than HEADROOM gets a
      // new offset at once: its sum is rescaled by an exact power of two, this
      // tile's exponents subtract the shift (an exact integer subtraction), and
      // the query operand carries the new offset into the following tiles.
      // Weights stay below 2^64 of the offset, so the sums cannot overflow and
      // no chunk is ever redone (one extra VALU maximum per score, which these
      // MFMA-bound shapes absorb).  The first tile, and a jump of more than
      // 1024, score the tile again at the new offsets instead, so the exponent
      // keeps the rounding of a small magnitude.
      bool coarse = false;
#pragma unroll 1
      for (int t = 0; t < TC; ++t) {
        Acc acc[R];
        tile(buf, t, acc);
        const bool first = ci == c0 && t == 0;
        float dl[R];
        bool raise = false, again = first;
#pragma unroll
        for (int c = 0; c < R; ++c) {
          float mx = -INFINITY;
#pragma unroll
          for (int o = 0; o < NO; ++o) mx = fmaxf(mx, acc[c][o]);
          mx = lanes_max(mx);
          dl[c] = 0.f;
          if (first || mx > HEADROOM) {
            const float mn = first ? offset_from_max(mx + HEADROOM, qg, coarse)
                                   : fmaxf(m[c], offset_from_max(m[c] + mx + HEADROOM, qg, coarse));
            dl[c] = mn - m[c];
            s[c] = first ? 0.f : rescale(s[c], m[c], mn);
            m[c] = mn;
            set_offset(bq[c][0], -mn, grp == 0);
            raise = true;
            again |= !(mx <= 1024.f);
          }
        }
        if (__any(again)) {
          tile(buf, t, acc);
        } else if (__any(raise)) {
#pragma unroll
          for (int c = 0; c < R; ++c)
#pragma unroll
            for (int o = 0; o < NO; ++o) acc[c][o] -= dl[c];
        }
        accumulate(acc);
      }
      flag_if(status, coarse && lane == 0, FLAG_SCORE_RANGE);
      if (ci + 1 < c1) lstore(Par<P ^ 1>{});
      __syncthreads();
      return;
    }

    float ssave[R];
#pragma unroll
    for (int c = 0; c < R; ++c) ssave[c] = s[c];

    if (ci == c0) {
      // First offsets: the maximum raw score of the chunk's first key tile plus
      // HEADROOM, so later keys may score up to HEADROOM + 112 higher before a
      // chunk has to be redone.
      if (MODE == MODE_SPLIT) {
#pragma unroll
        for (int c = 0; c < R; ++c) set_offset(bq[c][0], 0.f, grp == 0);
      }
      Acc acc[R];
      tile(buf, 0, acc);
      bool coarse = false;
#pragma unroll
      for (int c = 0; c < R; ++c) {
        float mx = -INFINITY;
#pragma unroll
        for (int o = 0; o < NO; ++o) mx = fmaxf(mx, raw(acc[c][o]));
        m[c] = offset_from_max(lanes_max(mx) + HEADROOM, qg, coarse);
        if (MODE == MODE_SPLIT) set_offset(bq[c][0], -m[c], grp == 0);
      }
      flag_if(status, coarse && lane == 0, FLAG_SCORE_RANGE);
    }
    if constexpr (NCH == 1) {
      // short K: the unrolled tiles let the scheduler overlap one tile's MFMAs
      // with the previous tile's exps (about 1% at d <= 3; larger K spills)
#pragma unroll
      for (int t = 0; t < TC; ++t) {
        Acc acc[R];
        tile(buf, t, acc);
        accumulate(acc);
      }
    } else {
#pragma unroll 1
      for (int t = 0; t < TC; ++t) {
        Acc acc[R];
        tile(buf, t, acc);
        accumulate(acc);
      }
    }
    int bad = 0;
#pragma unroll
    for (int c = 0; c < R; ++c) bad |= !(s[c] <= SUM_LIMIT);
    const bool redo = __any(bad);
    if (redo) {
      // Exact chunk maximum of the raw scores (offset slots zeroed), a new
      // offset from it, then the chunk again through the normal path.
#pragma unroll
      for (int c = 0; c < R; ++c) s[c] = ssave[c];
      if (MODE == MODE_SPLIT) {
#pragma unroll
        for (int c = 0; c < R; ++c) set_offset(bq[c][0], 0.f, grp == 0);
      }
      float mx[R];
#pragma unroll
      for (int c = 0; c < R; ++c) mx[c] = -INFINITY;
#pragma unroll 1
      for (int t = 0; t < TC; ++t) {
        Acc acc[R];
        tile(buf, t, acc);
#pragma unroll
        for (int c = 0; c < R; ++c)
#pragma unroll
          for (int o = 0; o < NO; ++o) mx[c] = fmaxf(mx[c], raw(acc[c][o]));
      }
      bool coarse = false;
#pragma unroll
      for (int c = 0; c < R; ++c) {
        mx[c] = lanes_max(mx[c]);
        const float mn = fmaxf(m[c], offset_from_max(mx[c] + HEADROOM, qg, coarse));
        s[c] = rescale(s[c], m[c], mn);
        m[c] = mn;
        if (MODE == MODE_SPLIT) set_offset(bq[c][0], -m[c], grp == 0);
      }
      flag_if(status, coarse && lane == 0, FLAG_SCORE_RANGE);
#pragma unroll 1
      for (int t = 0; t < TC; ++t) {
        Acc acc[R];
        tile(buf, t, acc);
        accumulate(acc);
      }
    }
    if (ci + 1 < c1) lstore(Par<P ^ 1>{});
    __syncthreads();
  };

  if (c0 < c1) {
    gload(c0, Par<0>{});
    lstore(Par<0>{});
    __syncthreads();
    for (int ci = c0; ci < c1; ci += 2) {
      step(ci, Par<0>{});
      if (ci + 1 < c1) step(ci + 1, Par<1>{});
    }
  }  // c0 < c1 (an empty key range leaves m = -FLT_MAX, s = 0: a neutral partial)

  if constexpr (WV) {
#pragma unroll
    for (int c = 0; c < R; ++c) {
      const float st = WV == 1 ? lanes_sum(s[c]) : 0.f, wt = lanes_sum(ws[c]);
      const int q = qbase + MW * c + col;
      if (grp == 0 && q < rows) part[(size_t)blk.y * batch * rows + (size_t)b * rows + q] = make_float2(wt, st);
    }
    return;
  }

#pragma unroll
  for (int c = 0; c < R; ++c) {
    const float st = lanes_sum(s[c]);
    const int q = qbase + MW * c + col;
    if (grp == 0 && q < rows) {
      const size_t r = (size_t)b * rows + q;
      if (part != nullptr) {
        part[(size_t)blk.y * batch * rows + r] = make_float2(m[c], st);
      } else {
        const float v = (float)(qnorm[r] - ((double)m[c] + log2((double)st)) * inv_lam);
        out[r] = v;
        flag_if(status, !isfinite(v), FLAG_NONFINITE);
        if (nb.logw != nullptr) write_next_bias(nb, b, q, v, qnorm[r], nb.logw[r]);
      }
    }
  }
}


// Two packed bf16 parts of a weight pair: hi = e truncated to bf16 (its upper
// half), lo = rne(e - hi), where e - hi is exact; together 16 significant bits.
// Returns (hi pair, lo pair).  The hi pair is one byte permute; e - hi is one
// bf16 dot product each, hi . (-1, -0) + a and hi . (0, -1) + b (products and
// sums exact).  The first pair is written (-1, -0) so that it is encoded as a
// 32-bit literal: hipcc encodes (-1, 0) as the inline constant -1.0, which
// this instruction reads as the fp32 bit pattern, i.e. as the pair (0, -1).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 split_pair(float a, float b) {
  const uint32_t hi = __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
  const bf16x2 h = __builtin_bit_cast(bf16x2, hi);
  const float la = __builtin_amdgcn_fdot2_f32_bf16(h, bf16x2{(__bf16)-1.f, (__bf16)-0.f}, a, false);
  const float lb = __builtin_amdgcn_fdot2_f32_bf16(h, bf16x2{(__bf16)0.f, (__bf16)-1.f}, b, false);
  const bf16x2 l = {(__bf16)la, (__bf16)lb};
  return make_uint2(hi, __builtin_bit_cast(uint32_t, l));
}

// ---------------------------------------------------------------------------
// Wide operands: the half-step with a K loop (fp32 inputs with d > 88 in the
// hi/lo layout; bf16 inputs with d > 256).  The query operand no longer fits
// in registers, so both operands pass through LDS in chunks of 32 K slots, and
// each workgroup keeps a 256-query x 256-key block of scores in registers:
// eight waves in a 4 x 2 arrangement, each 64 queries x 128 keys (2 x 4 tiles
// of v_mfma_f32_32x32x16_bf16, 128 accumulators per lane).  A 16-slot step
// reads 6 fragments for 8 MFMAs.  When a key block's scores are complete, each
// query's exact block maximum (its two lanes combined) moves the running
// offset only when it passes it, so no block is ever recomputed, then the
// block's exponentials are summed.  The two key halves of a query (two waves)
// are merged through LDS at the end; key splits go to k_merge as usual.
//   hi/lo: acc starts at lambda*beta_j and adds 2 lambda x.y from the products
//          x_h v_h + x_h v_l + x_l v_h (sc = 1);
//   bf16:  acc starts at beta_j / 2 and adds x.y (sc = 2 lambda).
// The exponent is fma(acc, sc, -m).
//
// The same blocked product serves the wide plan passes (transport, plan
// application, the HVP's row-weighted pass), which go through a weights buffer
// holding one block of rows against all keys (the value product at these widths
// is compute bound many times over the buffer's traffic):
//   EPI_W:    the row block's weights 2^(score - M_i), M_i = lambda (|x_i|^2 - T_i)
//             from the row's half-step value T_i (so a row's weights sum to 1),
//             written as bf16 hi/lo parts, and their sums per key split;
//   EPI_U:    with the direction planes as rows and no bias, u_ij = ugain * acc
//             = (y_j - c) . v_i; the buffered weights are multiplied by u_ij;
//   EPI_GEMM: rows = weight rows (K = hi keys then lo keys), columns = value
//             columns (K wraps over the keys once), partial products per K split.
// In the weights buffer the 32 keys of a tile sit in the order in which a lane
// holds them (position 16 grp + o is key key_of(o, grp)); the value rows use the
// same order, so a lane moves its 16 weights as two 16-byte vectors.
// ---------------------------------------------------------------------------
constexpr int KL_NW = 8, KL_WQ = 4, KL_QT = 2, KL_KT = 4;
constexpr int KL_BQ = KL_WQ * KL_QT * 32;              // 256 queries per workgroup
constexpr int KL_BK = (KL_NW / KL_WQ) * KL_KT * 32;    // 256 keys per block
constexpr int KL_KC = 32;                               // K slots per LDS chunk
constexpr int KL_LR = KL_KC + 8;                        // LDS row stride (elements)
static_assert(ROW_PAD % KL_BQ == 0 && ROW_PAD % KL_BK == 0, "blocks must tile the row padding");
constexpr int EPI_LSE = 0, EPI_W = 1, EPI_U = 2, EPI_GEMM = 3;

// Key of position p (0..31) of a 32-key tile in the lane order of the weights.
__host__ __device__ constexpr int lane_key(int p) { return 8 * ((p % 16) / 4) + 4 * (p / 16) + (p % 4); }

// Arguments of the K-looped kernel.  A (row operand): rows of a_ld elements,
// a_rows rows per problem, the launch's first row a_row0; K chunk kc reads
// chunk kc % a_nkc of plane kc / a_nkc (planes a_plane elements apart).
// B (column operand): rows of b_ld elements, b_rows per problem; K chunk kc
// reads chunk kc % b_nkc.  Rows of the launch are rows row0.. of the problem.
struct KlArgs {
  const u16* A;
  const u16* B;
  const float* hb;       // bias of the B rows (accumulator start), or nullptr for 0
  const double* qnorm;   // |x_i|^2 of the rows (LSE, W)
  const float* lse;      // half-step values of the rows (W)
  float* out;            // potential (LSE without splits)
  float2* part;          // (max, sum) per split (LSE with splits)
  u16* wt;               // weights buffer (W, U)
  float* pv;             // partial products [split][batch][prows][nc] (GEMM)
  float* sp;             // weight sums [split][batch][prows] (W)
  unsigned* tag;
  unsigned tag_val;
  unsigned* status;
  long long a_plane;
  int a_ld, a_rows, a_row0, a_nkc;
  int b_ld, b_rows, b_nkc;
  int rows, row0, keys;
  int prows;             // rows per (split, problem) of pv and sp, counted from row0
  int nkc;               // K chunks per key block (LSE, W, U)
  int per_split;         // key blocks (LSE, W, U) or K chunks (GEMM) per split
  int total_kc;          // K chunks in all (GEMM)
  int ncolt, nc;         // column blocks and stored columns (GEMM)
  int wt_ld, kcov, wt_rows;  // weights buffer: row stride, offset of the lo parts, rows per problem
  int batch;
  float sc, lam, ugain;
  double inv_lam;
  NextBias nb;
};

template <int EPI>
__global__ __launch_bounds__(64 * KL_NW) __attribute__((amdgpu_waves_per_eu(2))) void k_lsek(const KlArgs a) {
  using T = Tile<32>;
  using Acc = typename T::Acc;
  constexpr int NT = 64 * KL_NW;
  constexpr int ROWS = KL_BQ + KL_BK;                 // operand rows staged per chunk
  constexpr int SEGS = KL_KC / 8;                     // 16-byte segments per row and chunk
  constexpr int NLD = ROWS * SEGS / NT;               // 16-byte loads per thread per chunk
  static_assert(KL_KC % 16 == 0 && ROWS * SEGS % NT == 0, "whole K steps and whole loads per thread");
  __shared__ __attribute__((aligned(16))) u16 lds[2][ROWS * KL_LR];
  __shared__ float ldb[KL_BK];
  __shared__ float2 ldm[KL_BQ];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane >> 5, col = lane & 31;
  const int wq = wave % KL_WQ, wk = wave / KL_WQ;
  const int b = blockIdx.z;
  const int q0 = blockIdx.x * KL_BQ;  // first row of the workgroup within the launch
  if (a.tag != nullptr && tid == 0 && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0) *a.tag = a.tag_val;
  const u16* Ab = a.A + ((size_t)b * a.a_rows + a.a_row0 + q0) * a.a_ld;
  const u16* Bb = a.B + (size_t)b * a.b_rows * a.b_ld;
  const float* hbb = a.hb != nullptr ? a.hb + (size_t)b * a.b_rows : nullptr;
  int kb0, kb1, kc0, kc1;
  if (EPI == EPI_GEMM) {
    kb0 = blockIdx.y % a.ncolt;
    kb1 = kb0 + 1;
    kc0 = (blockIdx.y / a.ncolt) * a.per_split;
    kc1 = min(a.total_kc, kc0 + a.per_split);
  } else {
    const int nblk = (a.keys + KL_BK - 1) / KL_BK;
    kb0 = blockIdx.y * a.per_split;
    kb1 = min(nblk, kb0 + a.per_split);
    kc0 = 0;
    kc1 = a.nkc;
  }

  float m[KL_QT], s[KL_QT], Mrow[KL_QT];
#pragma unroll
  for (int c = 0; c < KL_QT; ++c) {
    m[c] = -FLT_MAX;
    s[c] = 0.f;
    Mrow[c] = 0.f;
    if (EPI == EPI_W) {
      const int q = a.row0 + q0 + wq * (KL_QT * 32) + c * 32 + col;
      if (q < a.rows) {
        const size_t r = (size_t)b * a.rows + q;
        const double M = (double)a.lam * (a.qnorm[r] - (double)a.lse[r]);
        Mrow[c] = fabs(M) < 1e30 ? (float)M : 0.f;
      }
    }
  }

  // staging: load i of thread tid takes 16-byte segment (tid + NT i) % SEGS of row
  // (tid + NT i) / SEGS (rows 0..BQ-1 the workgroup's A rows, then the block's B rows)
  u4 pre[NLD];
  auto gload = [&](int kb, int kc) {
    const long long aoff = (long long)(kc / a.a_nkc) * a.a_plane + (long long)(kc % a.a_nkc) * KL_KC;
    const int boff = (kc % a.b_nkc) * KL_KC;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int idx = tid + NT * i, row = idx / SEGS, seg = idx % SEGS;
      const u16* src = row < KL_BQ ? Ab + (size_t)row * a.a_ld + aoff
                                   : Bb + ((size_t)kb * KL_BK + (row - KL_BQ)) * a.b_ld + boff;
      pre[i] = *reinterpret_cast<const u4*>(src + seg * 8);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int idx = tid + NT * i, row = idx / SEGS, seg = idx % SEGS;
      *reinterpret_cast<u4*>(&lds[buf][row * KL_LR + seg * 8]) = pre[i];
    }
  };
  // the weights-buffer row of query tile c and the start of key tile t of block kb
  auto wrow = [&](int c, int kb, int t) {
    return a.wt + ((size_t)b * a.wt_rows + q0 + wq * (KL_QT * 32) + c * 32 + col) * a.wt_ld + (size_t)kb * KL_BK +
           wk * (KL_KT * 32) + t * 32 + grp * 16;
  };

  if (kb0 < kb1) {
    Acc acc[KL_QT][KL_KT];
    int buf = 0;
    if (kc0 < kc1) gload(kb0, kc0);
    if (hbb != nullptr && tid < KL_BK) ldb[tid] = hbb[(size_t)kb0 * KL_BK + tid];
    lstore(0);
    __syncthreads();
    for (int kb = kb0; kb < kb1; ++kb) {
      // accumulators start at the keys' bias
#pragma unroll
      for (int t = 0; t < KL_KT; ++t) {
        Acc ci;
#pragma unroll
        for (int o = 0; o < 16; ++o) ci[o] = hbb != nullptr ? ldb[wk * (KL_KT * 32) + t * 32 + T::key_of(o, grp)] : 0.f;
#pragma unroll
        for (int c = 0; c < KL_QT; ++c) acc[c][t] = ci;
      }
      float nbias = 0.f;
      for (int kc = kc0; kc < kc1; ++kc) {
        const bool more = kc + 1 < kc1 || kb + 1 < kb1;
        if (kc + 1 < kc1)
          gload(kb, kc + 1);
        else if (kb + 1 < kb1)
          gload(kb + 1, kc0);
        const bool nb_load = hbb != nullptr && kc + 1 == kc1 && kb + 1 < kb1 && tid < KL_BK;
        if (nb_load) nbias = hbb[(size_t)(kb + 1) * KL_BK + tid];
        const u16* L = lds[buf];
#pragma unroll
        for (int ks = 0; ks < KL_KC / 16; ++ks) {
          u4 bq[KL_QT];
#pragma unroll
          for (int c = 0; c < KL_QT; ++c)
            bq[c] = *reinterpret_cast<const u4*>(&L[(wq * (KL_QT * 32) + c * 32 + col) * KL_LR + ks * 16 + grp * 8]);
#pragma unroll
          for (int t = 0; t < KL_KT; ++t) {
            const u4 ka = *reinterpret_cast<const u4*>(
                &L[(KL_BQ + wk * (KL_KT * 32) + t * 32 + col) * KL_LR + ks * 16 + grp * 8]);
#pragma unroll
            for (int c = 0; c < KL_QT; ++c) acc[c][t] = T::mma(ka, bq[c], acc[c][t]);
          }
        }
        if (more) lstore(buf ^ 1);
        // the bias of the next block: every wave has read this block's at its start
        if (nb_load) ldb[tid] = nbias;
        __syncthreads();
        buf ^= 1;
      }
      if (EPI == EPI_LSE) {
        // block epilogue: exact block maximum, offset moves only past it, then the sums
        bool coarse = false;
#pragma unroll
        for (int c = 0; c < KL_QT; ++c) {
          float mx = -INFINITY;
#pragma unroll
          for (int t = 0; t < KL_KT; ++t)
#pragma unroll
            for (int o = 0; o < 16; ++o) mx = fmaxf(mx, acc[c][t][o] * a.sc);
          mx = fmaxf(mx, __shfl_xor(mx, 32));
          if (!(mx <= m[c])) {
            const float mn = fmaxf(m[c], offset_from_max(mx + HEADROOM, 1.f, coarse));
            s[c] = rescale(s[c], m[c], mn);
            m[c] = mn;
          }
          float e[16];
#pragma unroll
          for (int o = 0; o < 16; ++o) e[o] = 0.f;
#pragma unroll
          for (int t = 0; t < KL_KT; ++t)
#pragma unroll
            for (int o = 0; o < 16; ++o) e[o] += __builtin_amdgcn_exp2f(fmaf(acc[c][t][o], a.sc, -m[c]));
#pragma unroll
          for (int w = 1; w < 16; w *= 2)
#pragma unroll
            for (int o = 0; o + w < 16; o += 2 * w) e[o] += e[o + w];
          s[c] += e[0];
        }
        flag_if(a.status, coarse && lane == 0, FLAG_SCORE_RANGE);
      } else if (EPI == EPI_W || EPI == EPI_U) {
#pragma unroll
        for (int c = 0; c < KL_QT; ++c)
#pragma unroll
          for (int t = 0; t < KL_KT; ++t) {
            u16* wp = wrow(c, kb, t);
            float e[16];
            if (EPI == EPI_W) {
              float sum = 0.f;
#pragma unroll
              for (int o = 0; o < 16; ++o) {
                e[o] = __builtin_amdgcn_exp2f(fmaf(acc[c][t][o], a.sc, -Mrow[c]));
                sum += e[o];
              }
              s[c] += sum;
            } else {
              const u4 h0 = *reinterpret_cast<const u4*>(wp), h1 = *reinterpret_cast<const u4*>(wp + 8);
              const u4 l0 = *reinterpret_cast<const u4*>(wp + a.kcov), l1 = *reinterpret_cast<const u4*>(wp + a.kcov + 8);
              const uint32_t hw[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
              const uint32_t lw[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
#pragma unroll
              for (int h = 0; h < 8; ++h) {
                e[2 * h] = __uint_as_float(hw[h] << 16) + __uint_as_float(lw[h] << 16);
                e[2 * h + 1] = __uint_as_float(hw[h] & 0xffff0000u) + __uint_as_float(lw[h] & 0xffff0000u);
              }
#pragma unroll
              for (int o = 0; o < 16; ++o) e[o] *= acc[c][t][o] * a.ugain;
            }
            uint2 pr[8];
#pragma unroll
            for (int h = 0; h < 8; ++h) pr[h] = split_pair(e[2 * h], e[2 * h + 1]);
            *reinterpret_cast<u4*>(wp) = u4{pr[0].x, pr[1].x, pr[2].x, pr[3].x};
            *reinterpret_cast<u4*>(wp + 8) = u4{pr[4].x, pr[5].x, pr[6].x, pr[7].x};
            *reinterpret_cast<u4*>(wp + a.kcov) = u4{pr[0].y, pr[1].y, pr[2].y, pr[3].y};
            *reinterpret_cast<u4*>(wp + a.kcov + 8) = u4{pr[4].y, pr[5].y, pr[6].y, pr[7].y};
          }
      } else {
        // partial products: lane (row col, group grp) holds columns key_of(o, grp) of each tile
        const int split = blockIdx.y / a.ncolt;
#pragma unroll
        for (int c = 0; c < KL_QT; ++c) {
          const int ql = q0 + wq * (KL_QT * 32) + c * 32 + col;
          if (a.row0 + ql >= a.rows) continue;
          float* dst = a.pv + (((size_t)split * a.batch + b) * a.prows + ql) * a.nc;
#pragma unroll
          for (int t = 0; t < KL_KT; ++t)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const int cc = kb * KL_BK + wk * (KL_KT * 32) + t * 32 + 8 * u + 4 * grp;
              if (cc < a.nc)
                *reinterpret_cast<f4*>(dst + cc) =
                    f4{acc[c][t][4 * u], acc[c][t][4 * u + 1], acc[c][t][4 * u + 2], acc[c][t][4 * u + 3]};
            }
        }
      }
    }
  }
  if (EPI == EPI_LSE) {
    // the two lanes of a query share its offset; then the two key halves (waves
    // wk = 0, 1) merge through LDS
#pragma unroll
    for (int c = 0; c < KL_QT; ++c) s[c] += __shfl_xor(s[c], 32);
    if (wk == 1 && grp == 0) {
#pragma unroll
      for (int c = 0; c < KL_QT; ++c) ldm[wq * (KL_QT * 32) + c * 32 + col] = make_float2(m[c], s[c]);
    }
    __syncthreads();
    if (wk == 0 && grp == 0) {
#pragma unroll
      for (int c = 0; c < KL_QT; ++c) {
        const int ql = wq * (KL_QT * 32) + c * 32 + col;
        const float2 o = ldm[ql];
        const float M = fmaxf(m[c], o.x);
        const float S = rescale(s[c], m[c], M) + rescale(o.y, o.x, M);
        const int q = q0 + ql;
        if (q < a.rows) {
          const size_t r = (size_t)b * a.rows + q;
          if (a.part != nullptr) {
            a.part[(size_t)blockIdx.y * a.batch * a.rows + r] = make_float2(M, S);
          } else {
            const float v = (float)(a.qnorm[r] - ((double)M + log2((double)S)) * a.inv_lam);
            a.out[r] = v;
            flag_if(a.status, !isfinite(v), FLAG_NONFINITE);
            if (a.nb.logw != nullptr) write_next_bias(a.nb, b, q, v, a.qnorm[r], a.nb.logw[r]);
          }
        }
      }
    }
  } else if (EPI == EPI_W) {
    // weight sums of the split: both lanes of a row, then both key halves
#pragma unroll
    for (int c = 0; c < KL_QT; ++c) s[c] += __shfl_xor(s[c], 32);
    if (wk == 1 && grp == 0) {
#pragma unroll
      for (int c = 0; c < KL_QT; ++c) ldm[wq * (KL_QT * 32) + c * 32 + col] = make_float2(0.f, s[c]);
    }
    __syncthreads();
    if (wk == 0 && grp == 0) {
#pragma unroll
      for (int c = 0; c < KL_QT; ++c) {
        const int ql = wq * (KL_QT * 32) + c * 32 + col;
        if (a.row0 + q0 + ql < a.rows) a.sp[((size_t)blockIdx.y * a.batch + b) * a.prows + q0 + ql] = s[c] + ldm[ql].y;
      }
    }
  }
}

// Key rows of the hi/lo layout for one side: (v_h, v_l, v_h) per coordinate,
// v = 2 lambda (y - c) in two bf16 parts (fp64 arithmetic).  They depend only on
// the cloud and lambda: *tag holds the bit pattern of the lambda they were built
// for, a launch with the same lambda writes nothing, and a rebuild clears the
// tag (the half-step kernel that follows sets it).  One thread per 16-byte segment.
__global__ __launch_bounds__(256) void k_prep_keys_hilo(const void* __restrict__ P, int in_bf16,
                                                        const double* __restrict__ cen, int keys, int keys_pad,
                                                        int d, int KP, float lam, unsigned* __restrict__ tag,
                                                        u16* __restrict__ kb) {
  const int b = blockIdx.y;
  if (*tag == __float_as_uint(lam)) return;
  const long long gtid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gtid == 0 && b == 0) *tag = 0u;
  const int vpr = KP / 8;
  if (gtid >= (long long)keys_pad * vpr) return;
  const int j = (int)(gtid / vpr), k0 = (int)(gtid % vpr) * 8;
  const double l2 = 2.0 * (double)lam;
  u16 v8[8];
  for (int e = 0; e < 8; ++e) {
    const int k = k0 + e, t = k / 3;
    u16 h = 0;
    if (j < keys && t < d) {
      const double v = l2 * ((double)coord(P, ((size_t)b * keys + j) * d + t, in_bf16) - cen[(size_t)b * d + t]);
      const u16 vh = bf16_of(v);
      h = (k % 3 == 1) ? bf16_of(v - (double)bf16_f(vh)) : vh;
    }
    v8[e] = h;
  }
  *reinterpret_cast<u4*>(kb + ((size_t)b * keys_pad + j) * KP + k0) =
      u4{(uint32_t)v8[0] | ((uint32_t)v8[1] << 16), (uint32_t)v8[2] | ((uint32_t)v8[3] << 16),
         (uint32_t)v8[4] | ((uint32_t)v8[5] << 16), (uint32_t)v8[6] | ((uint32_t)v8[7] << 16)};
}

// Value rows of a wide plan pass, [batch][ncp][kcov] bf16 with the keys of each
// 32-key tile in lane order (lane_key).  Row cc: without M, the centred
// coordinates of the key cloud in `parts` bf16 parts (cc = part d + t; one part
// holds a bf16 input exactly, two parts hold 16 significant bits of an fp32 one,
// from fp64); with M, three parts of the fp32 matrix columns col0.. (cc = part cb
// + k, exact).  Other rows and padding keys are zero.  One thread per 8 positions.
__global__ __launch_bounds__(256) void k_prep_vt(const void* __restrict__ P, int in_bf16,
                                                 const double* __restrict__ cen, const float* __restrict__ M, int c,
                                                 int col0, int cb, int parts, int keys, int kcov, int d, int ncp,
                                                 u16* __restrict__ vt) {
  const int b = blockIdx.y;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int per_row = kcov / 8;
  if (idx >= (long long)ncp * per_row) return;
  const int cc = (int)(idx / per_row), p0 = (int)(idx % per_row) * 8;
  u16 v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int p = p0 + e, j = (p / 32) * 32 + lane_key(p % 32);
    u16 val = 0;
    if (j < keys && M != nullptr && cc < 3 * cb) {
      const float x = M[((size_t)b * keys + j) * c + col0 + cc % cb];
      const u16 h0 = bf16_rne(x);
      const float r1 = x - bf16_f(h0);
      const u16 h1 = bf16_rne(r1);
      const int part = cc / cb;
      val = part == 0 ? h0 : (part == 1 ? h1 : bf16_rne(r1 - bf16_f(h1)));
    } else if (j < keys && M == nullptr && cc < parts * d) {
      const int t = cc % d;
      const double x = (double)coord(P, ((size_t)b * keys + j) * d + t, in_bf16) - cen[(size_t)b * d + t];
      const u16 h = bf16_of(x);
      val = cc / d == 0 ? h : bf16_of(x - (double)bf16_f(h));
    }
    v[e] = val;
  }
  *reinterpret_cast<u4*>(vt + ((size_t)b * ncp + cc) * kcov + p0) = pack8(v);
}

// Merge the (max, sum) pairs of the key splits (one pass, exact power-of-two
// rescaling) and write the potential.
__global__ __launch_bounds__(256) void k_merge(const float2* __restrict__ part, int ks, int total, int rows,
                                               const double* __restrict__ qnorm, float* __restrict__ out,
                                               double inv_lam, unsigned* __restrict__ status, NextBias nb) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  // Two passes over the partials (the second from cache): the loads of a pass
  // are independent, so they overlap instead of waiting on a running offset.
  float M = -FLT_MAX, S = 0.f;
#pragma unroll 8
  for (int k = 0; k < ks; ++k) M = fmaxf(M, part[(size_t)k * total + i].x);
#pragma unroll 8
  for (int k = 0; k < ks; ++k) {
    const float2 v = part[(size_t)k * total + i];
    S += rescale(v.y, v.x, M);
  }
  const float v = (float)(qnorm[i] - ((double)M + log2((double)S)) * inv_lam);
  out[i] = v;
  flag_if(status, !isfinite(v), FLAG_NONFINITE);
  if (nb.logw != nullptr) write_next_bias(nb, i / rows, i % rows, v, qnorm[i], nb.logw[i]);
}

// sum_i exp(logw_i) * |expm1((pot_i - tilde_i)/eps)|, one workgroup per problem, fixed order.
__global__ __launch_bounds__(256) void k_marginal(const float* __restrict__ pot, const float* __restrict__ tilde,
                                                  const double* __restrict__ logw, int rows, float inv_eps,
                                                  float* __restrict__ err, int which) {
  __shared__ float red[256];
  const int b = blockIdx.x;
  float acc = 0.f;
  for (int i = threadIdx.x; i < rows; i += 256) {
    const size_t r = (size_t)b * rows + i;
    acc += (float)exp(logw[r]) * fabsf(expm1f((pot[r] - tilde[r]) * inv_eps));
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) err[2 * b + which] = red[0];
}

// ---------------------------------------------------------------------------
// Transport application (page "FlashSinkhorn: Trasporto Ottimo Entropico Consapevole delle I/O su GPU",
// section "Metodologia", part "3. Differenziazione e Ottimizzazione del Secondo Ordine"): the barycentric
// projection bary_i = sum_j P_ij y_j / sum_j P_ij and the gradient
// sum_j P_ij 2 (x_i - y_j) = 2 r_i (x_i - bary_i), r_i = sum_j P_ij, are
// softmax-weighted averages of the other cloud: an attention-style P.V product
// streamed over the same key chunks as the half-step, with V = the other
// cloud's coordinates and the plan never formed.
//
// MI355X design:
//  * The row offset is fixed before the pass: it is the row log-sum-exp that a
//    half-step computes first, so every weight is at most about 1, no running
//    maximum is kept and the partial sums of key splits simply add.
//  * The weights leave the score MFMA in its accumulator layout and enter the
//    P.V MFMA (16x16x32) as its A operand straight from registers: the keys of
//    V are read in the matching permuted order, so no shuffle or LDS round
//    trip is needed.  Two 16-key score tiles feed one 32-key P.V step.
//  * Each weight is split into two bf16 parts (16 significant bits) and each
//    fp32 coordinate into three bf16 parts (exact); bf16 coordinates are one
//    part.  The products are exact and accumulate in fp32; the final sums and
//    the division run in fp64.
// ---------------------------------------------------------------------------
// query tiles of 16 rows per wave, and waves per SIMD, of the transport kernel
// (nct value tiles of accumulators per query tile must fit beside the operands)
__host__ __device__ constexpr int bary_R(int nch, int nct) {
  return nct >= 9 ? 1 : (nch == 1 ? (nct >= 4 ? 2 : 4) : (nch <= 8 ? 2 : 1));
}
// 8 waves per workgroup share the staged key chunk, halving the key loads and
// LDS stores per query row.  Measured: plan products -21% at d = 32 (fp32),
// -8% at d = 128 (bf16); transport -3% at d = 128 (bf16) but +16% at d <= 3,
// which keeps 4.  Operands of 12 or more K chunks take 80-120 KB of LDS per
// workgroup (one per CU): there the registers allow two waves per SIMD only with
// at most 4 value tiles or the 13 of a 64-column plan product (other wide
// passes spill and keep 4 waves, one per SIMD).
__host__ __device__ constexpr bool bary_wide8(int mode, int nch, int nct, int nu) {
  return nu == 0 && (nch >= 12 ? (nct <= 4 || nct == 13) : (nch >= 9 || (mode == MODE_BF16 && nch >= 3)));
}
__host__ __device__ constexpr int bary_NW(int mode, int nch, int nct, int nu) {
  return bary_wide8(mode, nch, nct, nu) ? 8 : 4;
}
__host__ __device__ constexpr int bary_waves(int mode, int nch, int nct, int nu) {
  return nch >= 12 ? (bary_wide8(mode, nch, nct, nu) ? 2 : 1) : 2;
}
// 32-key value blocks per LDS chunk of the transport kernel (fewer barriers for
// small operands; two blocks for 3..10 K chunks with 6..8 value tiles, where the
// registers, not LDS, already hold one workgroup per CU: measured -4.7% per
// transport call at d = 128 bf16, -1.3% for 64 problems at d = 32; four blocks
// were slower, and for the one-tile plan products of the HVP's conjugate
// gradients two blocks halve the workgroups per CU: +33% per HVP)
__host__ __device__ constexpr int bary_TCB(int nch, int nct) {
  return (nch <= 2 && nct <= 4) ? 4 : ((nch >= 3 && nch <= 10 && nct >= 6 && nct <= 8) ? 2 : 1);
}


// Power-of-two scale that brings a cloud's centred coordinates, at most `amax`
// in magnitude, below 2^14: bf16 values times it are exact fp16 values (down to
// 2^-27 amax, below which they round, far under the transport's error bound).
__host__ __device__ inline float fp16_value_scale(float amax) {
  return amax > 0.f && amax < 3.0e38f ? ldexpf(1.f, 13 - ilogbf(amax)) : 1.f;
}
constexpr u16 F16_ONE = 0x3C00;

// Key order inside a 32-key value block: lane group g of the P.V MFMA takes the
// weights of keys 4g..4g+3 and 16+4g..16+4g+3 as its A operand, so those eight
// keys sit together at positions 8g..8g+7 and the lane reads its B operand as
// one 16-byte vector (two 8-byte reads of the plain order conflict on the LDS
// banks).  Element e of the 8-key vector at position k0 holds key vkey(k0, e).
__host__ __device__ constexpr int vkey(int k0, int e) { return (k0 / 8) * 4 + (e < 4 ? e : 12 + e); }

// Value operand of one cloud: per problem and 32-key block a [ncols][32] bf16
// tile, col = part*d + t (the LDS image of the block, keys in vkey order), and ones in the last
// column when it is spare (sumcol).  Padding keys and other columns are zero.
// One thread per 8 keys of one column.
// half_max != nullptr (bf16 inputs, transport pass): fp16 values scaled by
// fp16_value_scale(half_max[b]) and an fp16 ones column.
__global__ __launch_bounds__(256) void k_prep_vals(const void* __restrict__ P, int mode, int in_bf16,
                                                   const double* __restrict__ rnorm, const double* __restrict__ cen,
                                                   int keys, int keys_pad, int d, int ncols, int sumcol,
                                                   const float* __restrict__ half_max, u16* __restrict__ vt) {
  const int b = blockIdx.y;
  const long long per_blk = (long long)ncols * (VK / 8);
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)(keys_pad / VK) * per_blk) return;
  const int blk = (int)(idx / per_blk);
  const int rem = (int)(idx % per_blk);
  const int c = rem / (VK / 8), k0 = (rem % (VK / 8)) * 8;
  const int part = c / d, t = c % d;
  const float hs = half_max != nullptr ? fp16_value_scale(half_max[b]) : 1.f;
  u16 v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int j = blk * VK + vkey(k0, e);
    u16 val = 0;
    if (j < keys && sumcol && c == ncols - 1) {
      val = half_max != nullptr ? F16_ONE : BF16_ONE;
    } else if (j < keys && part < val_parts(mode)) {
      const size_t r = ((size_t)b * keys + j) * d + t;
      const double c = cen[(size_t)b * d + t];
      if (mode == MODE_BF16 && half_max != nullptr) {
        // x - c is a bf16 value (see k_bf16_exact); times a power of two it is an fp16 one
        const float x = (float)((double)bf16_f(static_cast<const u16*>(P)[r]) - c) * hs;
        val = __builtin_bit_cast(u16, (_Float16)x);
      } else if (mode == MODE_BF16) {
        val = bf16_rne((float)((double)bf16_f(static_cast<const u16*>(P)[r]) - c));  // exact (see k_bf16_exact)
      } else {
        // x = h0 + h1 + h2 exactly: each remainder is exact in fp32
        const float x = (float)((double)coord(P, r, in_bf16) * rnorm[(size_t)b * keys + j] - c);
        const u16 h0 = bf16_rne(x);
        const float r1 = x - bf16_f(h0);
        const u16 h1 = bf16_rne(r1);
        val = part == 0 ? h0 : (part == 1 ? h1 : bf16_rne(r1 - bf16_f(h1)));
      }
    }
    v[e] = val;
  }
  *reinterpret_cast<u4*>(vt + (((size_t)b * (keys_pad / VK) + blk) * ncols + c) * VK + k0) = pack8(v);
}

// One pass of P.V over a key range for 4 waves x R query tiles of 16 rows.
// Writes the partial weighted sums pv_out[split][b][row][NCT*16] (columns
// part*d + t, and the weight sums in the last column if SUMCOL) or, without
// SUMCOL, the partial weight sums to s_out[split][b][row].
// NU > 0: row-weighted values.  U holds NU query-layout planes of a per-row
// vector v_i (fp32 path: one split operand; bf16 path: hi and lo bf16 parts);
// the weights become P_ij * u_ij with u_ij = ugain * (key operand . U_i), i.e.
// u_ij = q_j . v_i, while s_out still sums the plain weights.
template <int MODE, int NCH, int NCT, bool SUMCOL, bool LAZY = false, int NU = 0>
__global__ __launch_bounds__(64 * bary_NW(MODE, NCH, NCT, NU))
    __attribute__((amdgpu_waves_per_eu(bary_waves(MODE, NCH, NCT, NU)))) void k_bary(
    const u16* __restrict__ Q, const u16* __restrict__ K, const float* __restrict__ hb, const u16* __restrict__ V,
    const float* __restrict__ qgrid, const double* __restrict__ qnorm, const float* __restrict__ lse,
    float* __restrict__ pv_out, float* __restrict__ s_out, int rows, int rows_pad, int keys, int keys_pad,
    int chunks_per_split, int batch, float lam, float lam2, float* __restrict__ m_out, unsigned* __restrict__ tag,
    unsigned tag_val, const u16* __restrict__ U, float ugain, unsigned* __restrict__ status) {
  constexpr int MW = 16, R = bary_R(NCH, NCT);
  using T = Tile<16>;
  constexpr int KP = NCH * 32;
  constexpr int NI = KP / T::KI;
  constexpr int LROW = KP + 16;  // 32-byte pad: conflict-free 16-wide operand reads
  constexpr int TCB = bary_TCB(NCH, NCT);  // value blocks per chunk
  constexpr int CK = TCB * VK;
  static_assert(ROW_PAD % CK == 0 && CK <= SLACK, "a key chunk must divide the row padding");
  constexpr int VPR = KP / 8;
  constexpr int NVEC = CK * VPR;
  constexpr int NW = bary_NW(MODE, NCH, NCT, NU), NT = 64 * NW;  // waves, threads per workgroup
  constexpr int NLD = (NVEC + NT - 1) / NT;
  constexpr int NC = NCT * 16;        // value columns
  constexpr int VROW = VK + 8;        // LDS row stride of the value tile (elements)
  constexpr int NVV = TCB * NC * (VK / 8);  // 16-byte vectors per chunk of value blocks
  constexpr int NLV = (NVV + NT - 1) / NT;
  constexpr int QPW = R * MW;
  // bf16 inputs, transport pass: fp16 weights (one P.V product instead of the
  // hi and lo bf16 parts) against fp16 values; the lazy offsets then keep every
  // weight below 2^15 and above 2^-24 of the largest (see the raise below)
  constexpr bool HALF = MODE == MODE_BF16 && LAZY && NU == 0;
  __shared__ __attribute__((aligned(16))) u16 lds[2][(CK + 1) * LROW];
  __shared__ __attribute__((aligned(16))) u16 ldv[2][(TCB * NC + 1) * VROW];
  __shared__ __attribute__((aligned(16))) float ldsb[2][CK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane / MW, col = lane % MW;
  const int b = blockIdx.z;
  const int qbase = blockIdx.x * (NW * QPW) + wave * QPW;
  const u16* Qb = Q + (size_t)b * rows_pad * KP;
  const u16* Kb = K + (size_t)b * keys_pad * KP;
  const u16* Vb = V + (size_t)b * keys_pad * NC;
  const float* hbb = (MODE == MODE_BF16) ? hb + (size_t)b * keys_pad : nullptr;
  const float qg = (MODE == MODE_SPLIT) ? qgrid[b] : 1.f;

  u4 bq[R][NI];
#pragma unroll
  for (int c = 0; c < R; ++c)
#pragma unroll
    for (int i = 0; i < NI; ++i)
      bq[c][i] = *reinterpret_cast<const u4*>(Qb + (size_t)(qbase + MW * c + col) * KP + i * T::KI + grp * 8);
  constexpr int NUP = NU > 0 ? NU : 1;
  u4 bu[NUP][R][NI];
  if (NU > 0) {
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int c = 0; c < R; ++c)
#pragma unroll
        for (int i = 0; i < NI; ++i)
          bu[u][c][i] = *reinterpret_cast<const u4*>(U + ((size_t)u * (batch * (size_t)rows_pad + SLACK) +
                                                          (size_t)b * rows_pad + qbase + MW * c + col) * KP +
                                                     i * T::KI + grp * 8);
  }

  // Fixed row offsets.  M = lam (||p||^2 - lse) is log2 of the row's sum of
  // 2^score, so every weight 2^(score - M) is at most about 1.  The fp32 path
  // carries the grid-aligned part of M in the query operand; the rest (below
  // the grid quantum) only scales a row's weights uniformly, which the
  // normalisation cancels, so it is subtracted on the VALU only when it could
  // be large enough to overflow the sums.
  float sub[R];
  // Lazy offsets (transport pass without a preceding half-step): mo is each
  // query's running offset (base 2), -inf before its first key.  On the fp32
  // path it also sits in the query operand; on the bf16 path it is sub.
  float mo[R];
  if (tag != nullptr && threadIdx.x == 0 && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0) *tag = tag_val;
#pragma unroll
  for (int c = 0; c < R; ++c) {
    mo[c] = -INFINITY;
    if (LAZY) {
      sub[c] = 0.f;
      if (MODE == MODE_SPLIT) set_offset(bq[c][0], 0.f, grp == 0);
      continue;
    }
    const int q = qbase + MW * c + col;
    double M = 0.0;
    if (q < rows) {
      const size_t r = (size_t)b * rows + q;
      M = (double)lam * (qnorm[r] - (double)lse[r]);
    }
    if (!(fabs(M) < 1e30)) M = 0.0;
    if (MODE == MODE_SPLIT) {
      bool coarse = false;
      const float mo = offset_from_max((float)M, qg, coarse);
      flag_if(status, coarse, FLAG_SCORE_RANGE);
      set_offset(bq[c][0], -mo, grp == 0);
      sub[c] = (float)(M - (double)mo);
    } else {
      sub[c] = (float)M;
    }
  }

  const int total_chunks = (keys + CK - 1) / CK;
  const int c0 = blockIdx.y * chunks_per_split;
  const int c1 = min(total_chunks, c0 + chunks_per_split);

  float s[R];
  f4 pv[R][NCT];
#pragma unroll
  for (int c = 0; c < R; ++c) {
    s[c] = 0.f;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) pv[c][ct] = f4{0.f, 0.f, 0.f, 0.f};
  }

  u4 pre[NLD];
  u4 prev[NLV];
  f4 preb = {0.f, 0.f, 0.f, 0.f};
  // Key rows past the end of a chunk land in the operand buffers' slack rows;
  // value vectors are clamped to the block; both store surplus to a spare row.
  auto gload = [&](int chunk) {
    const u16* src = Kb + (size_t)chunk * CK * KP;
#pragma unroll
    for (int i = 0; i < NLD; ++i) pre[i] = *reinterpret_cast<const u4*>(src + (size_t)(tid + NT * i) * 8);
    const u16* vsrc = Vb + (size_t)chunk * TCB * NC * VK;
#pragma unroll
    for (int i = 0; i < NLV; ++i) prev[i] = *reinterpret_cast<const u4*>(vsrc + (size_t)min(tid + NT * i, NVV - 1) * 8);
    if (MODE == MODE_BF16) preb = *reinterpret_cast<const f4*>(hbb + (size_t)chunk * CK + (tid % (CK / 4)) * 4);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int v = min(tid + NT * i, NVEC);
      *reinterpret_cast<u4*>(&lds[buf][(v / VPR) * LROW + (v % VPR) * 8]) = pre[i];
    }
#pragma unroll
    for (int i = 0; i < NLV; ++i) {
      const int v = min(tid + NT * i, NVV);
      *reinterpret_cast<u4*>(&ldv[buf][(v / (VK / 8)) * VROW + (v % (VK / 8)) * 8]) = prev[i];
    }
    if (MODE == MODE_BF16 && tid < CK / 4) *reinterpret_cast<f4*>(&ldsb[buf][tid * 4]) = preb;
  };
  // Scores of the 16-key tile t of the chunk against the R query tiles.
  // Scores of the 16-key tile t against the R query tiles; with NU > 0 also
  // the contraction of the same key rows with the U planes (into accu).
  auto score2 = [&](int buf, int t, f4 (&acc)[R], f4 (&accu)[R]) {
    f4 cinit = {0.f, 0.f, 0.f, 0.f};
    if (MODE == MODE_BF16) cinit = *reinterpret_cast<const f4*>(&ldsb[buf][t * MW + 4 * grp]);
#pragma unroll
    for (int c = 0; c < R; ++c) {
      acc[c] = cinit;
      accu[c] = f4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const u4 ka = *reinterpret_cast<const u4*>(&lds[buf][(t * MW + col) * LROW + i * T::KI + grp * 8]);
#pragma unroll
      for (int c = 0; c < R; ++c) {
        acc[c] = T::mma(ka, bq[c][i], acc[c]);
        if (NU > 0) {
#pragma unroll
          for (int u = 0; u < NU; ++u) accu[c] = T::mma(ka, bu[u][c][i], accu[c]);
        }
      }
    }
  };
  auto score = [&](int buf, int t, f4 (&acc)[R]) {
    f4 unused[R];
    score2(buf, t, acc, unused);
  };
  float sub_max = 0.f;
#pragma unroll
  for (int c = 0; c < R; ++c) sub_max = fmaxf(sub_max, sub[c]);
  const bool fine = (MODE == MODE_BF16) || (!LAZY && __any(!(sub_max <= 32.f)));

  auto pass = [&](auto fine_c) {
    constexpr bool FINE = decltype(fine_c)::value;
    auto weight = [&](float v, int c) -> float {
      if (MODE == MODE_BF16) return __builtin_amdgcn_exp2f(fmaf(v, lam2, -sub[c]));
      return __builtin_amdgcn_exp2f(FINE ? v - sub[c] : v);
    };
    gload(c0);
    lstore(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int ci = c0; ci < c1; ++ci) {
      const int buf = (ci - c0) & 1;
      if (ci + 1 < c1) gload(ci + 1);
#pragma unroll 1
      for (int vb = 0; vb < TCB; ++vb) {
      f4 a0[R], a1[R], u0[R], u1[R];
      score2(buf, 2 * vb, a0, u0);
      score2(buf, 2 * vb + 1, a1, u1);
      float e[R][8];
      auto weights = [&]() {
#pragma unroll
        for (int c = 0; c < R; ++c)
#pragma unroll
          for (int o = 0; o < 4; ++o) {
            e[c][o] = weight(a0[c][o], c);
            e[c][4 + o] = weight(a1[c][o], c);
          }
      };
      weights();
      if (LAZY) {
        // A weight above 2^32 (a score more than 32 above its query's offset),
        // or a query meeting its first keys, asks for a raise; the wave then
        // takes each query's block maximum, sets its offset HEADROOM above it,
        // rescales the sums and, on the fp32 path, scores the block again.
        // (Weights are non-negative: their bit patterns order like their
        // values, with NaN above all, so the maximum is an integer one.)
        uint32_t wm = 0u;
        bool first = false;
#pragma unroll
        for (int c = 0; c < R; ++c) {
          first |= mo[c] == -INFINITY;
#pragma unroll
          for (int o = 0; o < 8; ++o) wm = max(wm, __float_as_uint(e[c][o]));
        }
        if (__any(first || wm > __float_as_uint(HALF ? 0x1p15f : 0x1p32f))) {
          float mx[R];
#pragma unroll
          for (int c = 0; c < R; ++c) {
            float v = -INFINITY;
#pragma unroll
            for (int o = 0; o < 4; ++o) v = fmaxf(v, fmaxf(a0[c][o], a1[c][o]));
            mx[c] = v;
          }
#pragma unroll
          for (int c = 0; c < R; ++c) {
            float v = fmaxf(mx[c], __shfl_xor(mx[c], 16));
            v = fmaxf(v, __shfl_xor(v, 32));
            const float top = (MODE == MODE_BF16) ? v * lam2 : (mo[c] == -INFINITY ? v : mo[c] + v);
            float mn = mo[c];
            bool coarse = false;
            if (HALF) {
              // fp16 weights: an integer offset that puts the block maximum in
              // (2^13, 2^14] (the bf16 offset enters only through the exponent,
              // so it needs no bf16 parts)
              if (mo[c] == -INFINITY || !(top - mo[c] <= 15.f)) mn = fmaxf(mo[c], ceilf(top - 14.f));
              coarse = !(fabsf(top) < 0x1p22f);
            } else if (mo[c] == -INFINITY || !(top - mo[c] <= 32.f)) {
              mn = fmaxf(mo[c], offset_from_max(top + HEADROOM, qg, coarse));
            }
            flag_if(status, coarse, FLAG_SCORE_RANGE);
            if (!SUMCOL) s[c] = rescale(s[c], mo[c], mn);
            // P.V rows are queries 4grp+r; their offsets live in lanes col = 4grp+r
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float o_old = __shfl(mo[c], 4 * grp + r), o_new = __shfl(mn, 4 * grp + r);
#pragma unroll
              for (int ct = 0; ct < NCT; ++ct) pv[c][ct][r] = rescale(pv[c][ct][r], o_old, o_new);
            }
            mo[c] = mn;
            if (MODE == MODE_BF16) sub[c] = mn;
            if (MODE == MODE_SPLIT) set_offset(bq[c][0], -mn, grp == 0);
          }
          if (MODE == MODE_SPLIT) {
            score(buf, 2 * vb, a0);
            score(buf, 2 * vb + 1, a1);
          }
          weights();
        }
      }
      if constexpr (HALF) {
        // fp16 weights (round to nearest) as the A operand; their sums come from
        // the same rounded values (one dot product with (1, 1) per pair)
        u4 eh[R];
#pragma unroll
        for (int c = 0; c < R; ++c) {
          uint32_t w[4];
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const f16x2 pr = {(_Float16)e[c][2 * h], (_Float16)e[c][2 * h + 1]};
            w[h] = __builtin_bit_cast(uint32_t, pr);
            if (!SUMCOL) s[c] = __builtin_amdgcn_fdot2(pr, f16x2{(_Float16)1.f, (_Float16)1.f}, s[c], false);
          }
          eh[c] = u4{w[0], w[1], w[2], w[3]};
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const u4 vv = *reinterpret_cast<const u4*>(&ldv[buf][(vb * NC + ct * 16 + col) * VROW + 8 * grp]);
#pragma unroll
          for (int c = 0; c < R; ++c)
            pv[c][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, eh[c]),
                                                              __builtin_bit_cast(f16x8, vv), pv[c][ct], 0, 0, 0);
        }
        continue;
      }
      // A operand of the P.V step: lane (query col, group grp) holds the
      // weights of keys 4grp..4grp+3 of tile 0 and of tile 1, in that order.
      u4 ehi[R], elo[R];
#pragma unroll
      for (int c = 0; c < R; ++c) {
        if (!SUMCOL) s[c] += ((e[c][0] + e[c][1]) + (e[c][2] + e[c][3])) + ((e[c][4] + e[c][5]) + (e[c][6] + e[c][7]));
        if (NU > 0) {
#pragma unroll
          for (int o = 0; o < 4; ++o) {
            e[c][o] *= u0[c][o] * ugain;
            e[c][4 + o] *= u1[c][o] * ugain;
          }
        }
        const uint2 p0 = split_pair(e[c][0], e[c][1]), p1 = split_pair(e[c][2], e[c][3]);
        const uint2 p2 = split_pair(e[c][4], e[c][5]), p3 = split_pair(e[c][6], e[c][7]);
        ehi[c] = u4{p0.x, p1.x, p2.x, p3.x};
        elo[c] = u4{p0.y, p1.y, p2.y, p3.y};
      }
      // B operand: lane (column col, group grp) reads the same keys of V.
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const u4 vv = *reinterpret_cast<const u4*>(&ldv[buf][(vb * NC + ct * 16 + col) * VROW + 8 * grp]);
#pragma unroll
        for (int c = 0; c < R; ++c) {
          pv[c][ct] = T::mma(ehi[c], vv, pv[c][ct]);
          pv[c][ct] = T::mma(elo[c], vv, pv[c][ct]);
        }
      }
      }  // value blocks of the chunk
      if (ci + 1 < c1) lstore(buf ^ 1);
      __syncthreads();
    }
  };
  if (c0 < c1) {
    if (fine)
      pass(std::true_type{});
    else
      pass(std::false_type{});
  }

  const size_t split_base = (size_t)blockIdx.y * batch * rows + (size_t)b * rows;
#pragma unroll
  for (int c = 0; c < R; ++c) {
    float st = s[c];
#pragma unroll
    for (int w = MW; w < 64; w *= 2) st += __shfl_xor(st, w);
    const int q = qbase + MW * c + col;
    if (!SUMCOL && grp == 0 && q < rows) s_out[split_base + q] = st;
    if (LAZY && grp == 0 && q < rows) m_out[split_base + q] = mo[c];
    // P.V output: lane (column col, group grp), element r = query 4grp + r
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int qr = qbase + MW * c + 4 * grp + r;
      if (qr < rows) {
        float* dst = pv_out + (split_base + qr) * NC + col;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) dst[ct * 16] = pv[c][ct][r];
      }
    }
  }
}

// Rows of a merge: output rows row0 .. row0 + nrows of each problem (`rows`
// rows per problem in the outputs); the split partials hold prows rows per
// (split, problem), starting at row row0.  Weight sums: ks_s splits of sp, or
// with ks_s = 0 the ones column (the last) of the P.V partials.
struct MergeRows {
  int rows, row0, nrows, prows, ks_s;
};

// Barycentric projection and gradient from the split partials, one thread per
// (problem, row, coordinate): bary = sum_parts sum_splits pv / sum_splits s + c,
// grad = 2 r (p - bary) with the row mass r = w exp((pot - lse)/eps).
// With lazy offsets (mpart != nullptr; then ks_s is 0 or ks) each split's
// partials are relative to its own offset mpart (base 2): they are brought to
// the largest one, and the row's log-sum-exp follows from it and the weight
// sum, as in the half-step: lse = ||p||^2 - (M + log2 S) / lambda, written to
// lse for later passes.
__global__ __launch_bounds__(256) void k_bary_merge(const float* __restrict__ pv, const float* __restrict__ sp, int ks,
                                                    int batch, MergeRows mr, int d, int ncols, int parts,
                                                    const void* __restrict__ P, int in_bf16,
                                                    const float* __restrict__ pot, float* __restrict__ lse,
                                                    const double* __restrict__ logw, double eps,
                                                    const float* __restrict__ mpart, const double* __restrict__ qnorm,
                                                    double inv_lam, const double* __restrict__ cen,
                                                    const float* __restrict__ half_max, float* __restrict__ bary,
                                                    float* __restrict__ grad) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)batch * mr.nrows * d) return;
  const int t = (int)(idx % d);
  const int lr = (int)((idx / d) % mr.nrows), b = (int)(idx / ((long long)mr.nrows * d));
  const long long rr = (long long)b * mr.rows + mr.row0 + lr;  // b * rows + row
  const size_t pr = (size_t)b * mr.prows + lr;                 // row of the partials within a split
  const size_t pstride = (size_t)batch * mr.prows;
  double M = 0.0;
  if (mpart != nullptr) {
    M = -INFINITY;
#pragma unroll 4
    for (int k = 0; k < ks; ++k) M = fmax(M, (double)mpart[k * pstride + pr]);
  }
  double S = 0.0, num = 0.0;
#pragma unroll 4
  for (int k = 0; k < ks; ++k) {
    const size_t base = k * pstride + pr;
    const double sc = mpart != nullptr ? exp2((double)mpart[base] - M) : 1.0;  // 0 for an empty split
    if (mr.ks_s == 0) S += sc * (double)pv[base * ncols + ncols - 1];
    for (int part = 0; part < parts; ++part) num += sc * (double)pv[base * ncols + part * d + t];
  }
  for (int k = 0; k < mr.ks_s; ++k) {
    const size_t base = k * pstride + pr;
    S += (mpart != nullptr ? exp2((double)mpart[base] - M) : 1.0) * (double)sp[base];
  }
  const size_t o = (size_t)rr * d + t;
  // fp16 values carry a power-of-two scale (half_max: the key cloud's extent)
  if (half_max != nullptr) num /= (double)fp16_value_scale(half_max[b]);
  // the values were centred: the projection moves back by the centre
  const double bc = num / S + cen[(size_t)b * d + t];
  bary[o] = (float)bc;
  double row_lse;
  if (mpart != nullptr) {
    row_lse = qnorm[rr] - (M + log2(S)) * inv_lam;
    if (t == 0) lse[rr] = (float)row_lse;
  } else {
    row_lse = (double)lse[rr];
  }
  if (grad != nullptr) {
    const double x = coord(P, o, in_bf16);
    const double mass = exp(logw[rr] + ((double)pot[rr] - row_lse) / eps);
    grad[o] = (float)(2.0 * mass * (x - bc));
  }
}

// Cosine cost: the gradient in the raw point p from the barycentric projection
// of p_hat = p/|p| among the normalised points, by the chain rule through the
// normalisation: grad = (I - p_hat p_hat^T) 2 r (p_hat - bary) / |p|.  One
// thread per (problem, row); a zero point gets a zero gradient.
__global__ __launch_bounds__(256) void k_cosine_grad(const float* __restrict__ bary, const void* __restrict__ P,
                                                     int in_bf16, const double* __restrict__ rnorm,
                                                     const float* __restrict__ pot, const float* __restrict__ lse,
                                                     const double* __restrict__ logw, double eps, long long total,
                                                     int d, float* __restrict__ grad) {
  const long long rr = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (rr >= total) return;
  const double rn = rnorm[rr];
  const double mass = exp(logw[rr] + ((double)pot[rr] - (double)lse[rr]) / eps);
  double radial = 0.0;  // p_hat . (p_hat - bary)
  for (int t = 0; t < d; ++t) {
    const double ph = (double)coord(P, (size_t)rr * d + t, in_bf16) * rn;
    radial += ph * (ph - (double)bary[rr * d + t]);
  }
  for (int t = 0; t < d; ++t) {
    const double ph = (double)coord(P, (size_t)rr * d + t, in_bf16) * rn;
    const double gh = 2.0 * mass * (ph - (double)bary[rr * d + t]);
    grad[rr * d + t] = (float)((gh - radial * 2.0 * mass * ph) * rn);
  }
}

// ---------------------------------------------------------------------------
// Plan application and Hessian-vector products (page "FlashSinkhorn: Trasporto Ottimo Entropico
// Consapevole delle I/O su GPU", section "Metodologia", part "3. Differenziazione e Ottimizzazione
// del Secondo Ordine": the Hessian-vector product decomposes into vector- and
// matrix-transport products, so neither the Hessian nor the plan is formed).
// A plan application out_i = sum_j P_ij V_j is the transport pass above with V
// an arbitrary fp32 matrix, scaled by the row mass.
// ---------------------------------------------------------------------------

// Value operand from columns col0 .. col0+cb-1 of an fp32 matrix M [B][keys][c]:
// three exact bf16 parts per column (col = part*cb + k) and ones in the last
// column, keys in vkey order within each 32-key block.  One thread per 8 keys
// of one column.
__global__ __launch_bounds__(256) void k_prep_mat(const float* __restrict__ M, int keys, int keys_pad, int c, int col0,
                                                  int cb, int ncols, u16* __restrict__ vt) {
  const int b = blockIdx.y;
  const long long per_blk = (long long)ncols * (VK / 8);
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)(keys_pad / VK) * per_blk) return;
  const int blk = (int)(idx / per_blk);
  const int rem = (int)(idx % per_blk);
  const int cc = rem / (VK / 8), k0 = (rem % (VK / 8)) * 8;
  u16 v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int j = blk * VK + vkey(k0, e);
    u16 val = 0;
    if (j < keys && cc == ncols - 1) {
      val = BF16_ONE;
    } else if (j < keys && cc < 3 * cb) {
      const int part = cc / cb, k = cc % cb;
      const float x = M[((size_t)b * keys + j) * c + col0 + k];
      const u16 h0 = bf16_rne(x);
      const float r1 = x - bf16_f(h0);
      const u16 h1 = bf16_rne(r1);
      val = part == 0 ? h0 : (part == 1 ? h1 : bf16_rne(r1 - bf16_f(h1)));
    }
    v[e] = val;
  }
  *reinterpret_cast<u4*>(vt + (((size_t)b * (keys_pad / VK) + blk) * ncols + cc) * VK + k0) = pack8(v);
}

// out[b][row][col0+k] = r_row * (weighted sum of column k) / (sum of weights),
// r_row = w exp((pot - lse)/eps) the row mass.  One thread per (problem, row, k).
__global__ __launch_bounds__(256) void k_apply_merge(const float* __restrict__ pv, const float* __restrict__ sp, int ks,
                                                     int batch, MergeRows mr, int cb, int ncols, int c, int col0,
                                                     const double* __restrict__ logw, const float* __restrict__ pot,
                                                     const float* __restrict__ lse, double eps,
                                                     float* __restrict__ out) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)batch * mr.nrows * cb) return;
  const int k = (int)(idx % cb);
  const int lr = (int)((idx / cb) % mr.nrows), b = (int)(idx / ((long long)mr.nrows * cb));
  const long long rr = (long long)b * mr.rows + mr.row0 + lr;
  const size_t pr = (size_t)b * mr.prows + lr, pstride = (size_t)batch * mr.prows;
  double S = 0.0, num = 0.0;
#pragma unroll 4
  for (int q = 0; q < ks; ++q) {
    const size_t base = (q * pstride + pr) * ncols;
    if (mr.ks_s == 0) S += (double)pv[base + ncols - 1];
    for (int part = 0; part < 3; ++part) num += (double)pv[base + part * cb + k];
  }
  for (int q = 0; q < mr.ks_s; ++q) S += (double)sp[q * pstride + pr];
  const double mass = exp(logw[rr] + ((double)pot[rr] - (double)lse[rr]) / eps);
  out[rr * c + col0 + k] = (float)(mass > 0.0 ? mass * num / S : 0.0);
}

// One-vector plan product from the weighted half-step's split partials (W, S),
// one thread per (problem, row): out = r sum W / sum S with the row mass
// r = w exp((pot - lse)/eps) (the plan's row sums), as in k_apply_merge.
// mode 1 also stores r / sum S per row in scale; mode 2 takes that factor from
// scale (partials without sums): out = sum W * scale.
__global__ __launch_bounds__(256) void k_wv_merge(const float2* __restrict__ part, int ks, int batch, int rows,
                                                  const double* __restrict__ logw, const float* __restrict__ pot,
                                                  const float* __restrict__ lse, double eps, int mode,
                                                  double* __restrict__ scale, float* __restrict__ out) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long total = (long long)batch * rows;
  if (idx >= total) return;
  double W = 0.0, S = 0.0;
  for (int q = 0; q < ks; ++q) {
    const float2 v = part[q * total + idx];
    W += (double)v.x;
    S += (double)v.y;
  }
  if (mode == 2) {
    out[idx] = (float)(W * scale[idx]);
    return;
  }
  const double mass = exp(logw[idx] + ((double)pot[idx] - (double)lse[idx]) / eps);
  if (mode == 1) {
    const double sc = (mass > 0.0 && S > 0.0) ? mass / S : 0.0;
    scale[idx] = sc;
    out[idx] = (float)(W * sc);
    return;
  }
  out[idx] = (float)(mass > 0.0 ? mass * W / S : 0.0);
}

// Row masses r = w exp((pot - lse)/eps).
__global__ __launch_bounds__(256) void k_mass(const double* __restrict__ logw, const float* __restrict__ pot,
                                              const float* __restrict__ lse, double eps, long long total,
                                              double* __restrict__ mass) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < total) mass[i] = exp(logw[i] + ((double)pot[i] - (double)lse[i]) / eps);
}

// HVP set-up per row of the moving cloud (points p, direction v, PY = P Y):
//   z = p.v,  cr = 2 (r z - v.PY)  (= sum_j P_ij dC_ij),  and the matrix [z, v, cr/r]
// that the other side's plan application turns into the right-hand side.
__global__ __launch_bounds__(256) void k_hvp_rows(const void* __restrict__ P, int in_bf16, const float* __restrict__ V,
                                                  const float* __restrict__ PY, const double* __restrict__ mass,
                                                  long long total, int d, int rows, const double* __restrict__ cen,
                                                  double* __restrict__ zr, double* __restrict__ cr,
                                                  float* __restrict__ M) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  double z = 0.0, vpy = 0.0;
  for (int t = 0; t < d; ++t) {
    const double v = V[i * d + t];
    z += ccoord(P, (size_t)i, t, d, in_bf16, cen, (int)(i / rows)) * v;
    vpy += v * (double)PY[i * d + t];
  }
  const double r = mass[i];
  const double c = 2.0 * (r * z - vpy);
  zr[i] = z;
  cr[i] = c;
  float* row = M + i * (d + 2);
  row[0] = (float)z;
  for (int t = 0; t < d; ++t) row[1 + t] = V[i * d + t];
  row[d + 1] = (float)(r > 0.0 ? c / r : 0.0);
}

// Right-hand side of the Schur system per row of the fixed cloud (points q):
//   rhs = 2 (W0 - q.W1) - W2  with W = P^T [z, v, cr/r].
__global__ __launch_bounds__(256) void k_hvp_rhs(const void* __restrict__ Q, int in_bf16, const float* __restrict__ W,
                                                 long long total, int d, int keys, const double* __restrict__ cen,
                                                 double* __restrict__ rhs) {
  const long long j = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= total) return;
  const float* w = W + j * (d + 2);
  double qw = 0.0;
  for (int t = 0; t < d; ++t) qw += ccoord(Q, (size_t)j, t, d, in_bf16, cen, (int)(j / keys)) * (double)w[1 + t];
  rhs[j] = 2.0 * ((double)w[0] - qw) - (double)w[d + 1];
}

// Conjugate gradients on the Schur system (diag(c) - P^T diag(1/r) P) dg = rhs,
// preconditioned by diag(c), for every problem at once.  The system is singular
// along constants (a common shift of the potentials leaves the plan
// unchanged); the residual is kept at zero sum.  Each vector is split into
// CG_BLK-element blocks, one workgroup each; every reduction writes one partial
// per block and the next kernel adds the partials in block order (identical in
// every workgroup, so the result is deterministic).  Scalars per problem live
// in st[b][0..3] = (rz, rz0, done, pAp); rz is double buffered (st_in/st_out)
// because the kernel that computes the new value also reads the old one.

__device__ __forceinline__ double block_sum(double v, double* red) {
  __syncthreads();
  red[threadIdx.x] = v;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  return red[0];
}

// Sum of the nblk partials of problem b, in order.
__device__ __forceinline__ double sum_partials(const double* part, int nblk, double* red) {
  double v = 0.0;
  for (int k = threadIdx.x; k < nblk; k += 256) v += part[k];
  return block_sum(v, red);
}

// res = rhs, partial sums of res
__global__ __launch_bounds__(256) void k_cg_init1(const double* __restrict__ rhs, int m, int nblk,
                                                  double* __restrict__ res, double* __restrict__ part) {
  __shared__ double red[256];
  const int b = blockIdx.y;
  const size_t o = (size_t)b * m;
  const int j0 = blockIdx.x * CG_BLK, j1 = min(m, j0 + CG_BLK);
  double v = 0.0;
  for (int j = j0 + threadIdx.x; j < j1; j += 256) {
    res[o + j] = rhs[o + j];
    v += rhs[o + j];
  }
  v = block_sum(v, red);
  if (threadIdx.x == 0) part[(size_t)b * nblk + blockIdx.x] = v;
}

// res -= mean, z = res/c, pd = z, dg = 0, partials of res.z
__global__ __launch_bounds__(256) void k_cg_init2(const double* __restrict__ cmass, int m, int nblk,
                                                  const double* __restrict__ psum, double* __restrict__ dg,
                                                  double* __restrict__ res, double* __restrict__ pd,
                                                  float* __restrict__ pdf, double* __restrict__ part) {
  __shared__ double red[256];
  const int b = blockIdx.y;
  const size_t o = (size_t)b * m;
  const double mean = sum_partials(psum + (size_t)b * nblk, nblk, red) / m;
  const int j0 = blockIdx.x * CG_BLK, j1 = min(m, j0 + CG_BLK);
  double v = 0.0;
  for (int j = j0 + threadIdx.x; j < j1; j += 256) {
    const double r = res[o + j] - mean;
    const double z = cmass[o + j] > 0.0 ? r / cmass[o + j] : 0.0;
    res[o + j] = r;
    pd[o + j] = z;
    pdf[o + j] = (float)z;
    dg[o + j] = 0.0;
    v += r * z;
  }
  v = block_sum(v, red);
  if (threadIdx.x == 0) part[(size_t)b * nblk + blockIdx.x] = v;
}

// rz0 = rz = sum of the partials; done if zero
__global__ __launch_bounds__(256) void k_cg_init3(int nblk, const double* __restrict__ prz,
                                                  double* __restrict__ st) {
  __shared__ double red[256];
  const int b = blockIdx.x;
  const double rz = sum_partials(prz + (size_t)b * nblk, nblk, red);
  if (threadIdx.x == 0) {
    st[4 * b] = rz;
    st[4 * b + 1] = rz;
    st[4 * b + 2] = rz > 0.0 ? 0.0 : 1.0;
  }
}

// t <- t / r (the plan product of the search direction, per row of the moving cloud)
__global__ __launch_bounds__(256) void k_div_mass(float* __restrict__ t, const double* __restrict__ mass,
                                                  long long total) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < total) t[i] = (float)(mass[i] > 0.0 ? (double)t[i] / mass[i] : 0.0);
}

// partials of pd . S pd, S pd = c pd - q  (q = P^T (P pd / r))
__global__ __launch_bounds__(256) void k_cg_a(const float* __restrict__ q, const double* __restrict__ cmass, int m,
                                              int nblk, const double* __restrict__ pd, double* __restrict__ part) {
  __shared__ double red[256];
  const int b = blockIdx.y;
  const size_t o = (size_t)b * m;
  const int j0 = blockIdx.x * CG_BLK, j1 = min(m, j0 + CG_BLK);
  double v = 0.0;
  for (int j = j0 + threadIdx.x; j < j1; j += 256) v += pd[o + j] * (cmass[o + j] * pd[o + j] - (double)q[o + j]);
  v = block_sum(v, red);
  if (threadIdx.x == 0) part[(size_t)b * nblk + blockIdx.x] = v;
}

// alpha = rz / pAp; dg += alpha pd; res -= alpha S pd; partial sums of res
__global__ __launch_bounds__(256) void k_cg_b(const float* __restrict__ q, const double* __restrict__ cmass, int m,
                                              int nblk, const double* __restrict__ ppap,
                                              const double* __restrict__ st, double* __restrict__ dg,
                                              double* __restrict__ res, const double* __restrict__ pd,
                                              double* __restrict__ part) {
  __shared__ double red[256];
  const int b = blockIdx.y;
  const size_t o = (size_t)b * m;
  const double pap = sum_partials(ppap + (size_t)b * nblk, nblk, red);
  const double* s4 = st + 4 * b;
  const double alpha = (s4[2] != 0.0 || !(pap > 0.0)) ? 0.0 : s4[0] / pap;
  const int j0 = blockIdx.x * CG_BLK, j1 = min(m, j0 + CG_BLK);
  double v = 0.0;
  for (int j = j0 + threadIdx.x; j < j1; j += 256) {
    const double sp = cmass[o + j] * pd[o + j] - (double)q[o + j];
    dg[o + j] += alpha * pd[o + j];
    res[o + j] -= alpha * sp;
    v += res[o + j];
  }
  v = block_sum(v, red);
  if (threadIdx.x == 0) part[(size_t)b * nblk + blockIdx.x] = v;
}

// res -= mean; partials of res . z, z = res / c
__global__ __launch_bounds__(256) void k_cg_c(const double* __restrict__ cmass, int m, int nblk,
                                              const double* __restrict__ psum, double* __restrict__ res,
                                              double* __restrict__ part) {
  __shared__ double red[256];
  const int b = blockIdx.y;
  const size_t o = (size_t)b * m;
  const double mean = sum_partials(psum + (size_t)b * nblk, nblk, red) / m;
  const int j0 = blockIdx.x * CG_BLK, j1 = min(m, j0 + CG_BLK);
  double v = 0.0;
  for (int j = j0 + threadIdx.x; j < j1; j += 256) {
    const double r = res[o + j] - mean;
    res[o + j] = r;
    v += r * (cmass[o + j] > 0.0 ? r / cmass[o + j] : 0.0);
  }
  v = block_sum(v, red);
  if (threadIdx.x == 0) part[(size_t)b * nblk + blockIdx.x] = v;
}

// rz_new from the partials; stop test; pd = z + beta pd.  Reads st_in, writes st_out.
__global__ __launch_bounds__(256) void k_cg_d(const double* __restrict__ cmass, int m, int nblk,
                                              const double* __restrict__ prz, const double* __restrict__ ppap,
                                              double tol2, const double* __restrict__ st_in,
                                              double* __restrict__ st_out, const double* __restrict__ res,
                                              double* __restrict__ pd, float* __restrict__ pdf) {
  __shared__ double red[256];
  const int b = blockIdx.y;
  const size_t o = (size_t)b * m;
  const double rzn = sum_partials(prz + (size_t)b * nblk, nblk, red);
  const double pap = sum_partials(ppap + (size_t)b * nblk, nblk, red);
  const double* si = st_in + 4 * b;
  const bool stalled = !(pap > 0.0);
  const bool stop = si[2] != 0.0 || stalled || rzn <= tol2 * si[1];
  const double beta = stop ? 0.0 : rzn / si[0];
  const int j0 = blockIdx.x * CG_BLK, j1 = min(m, j0 + CG_BLK);
  for (int j = j0 + threadIdx.x; j < j1; j += 256) {
    const double z = cmass[o + j] > 0.0 ? res[o + j] / cmass[o + j] : 0.0;
    const double p = stop ? 0.0 : z + beta * pd[o + j];
    pd[o + j] = p;
    pdf[o + j] = (float)p;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    double* so = st_out + 4 * b;
    so[0] = si[2] != 0.0 ? si[0] : rzn;
    so[1] = si[1];
    so[2] = stop ? 1.0 : 0.0;
  }
}

// Matrix [dg, dg * q] per row of the fixed cloud (points q).
__global__ __launch_bounds__(256) void k_hvp_gmat(const void* __restrict__ Q, int in_bf16,
                                                  const double* __restrict__ dg, long long total, int d, int keys,
                                                  const double* __restrict__ cen, float* __restrict__ M) {
  const long long j = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= total) return;
  float* row = M + j * (d + 1);
  row[0] = (float)dg[j];
  for (int t = 0; t < d; ++t) row[1 + t] = (float)(dg[j] * ccoord(Q, (size_t)j, t, d, in_bf16, cen, (int)(j / keys)));
}

// Query-layout planes of a per-row fp32 vector v (the direction of a
// Hessian-vector product) for the row-weighted plan pass.  fp32 path: the
// points' split layout of v (grid part on a per-row quantum, two bf16
// remainders, in the same slots) with zeros in the offset and bias slots, so
// the key operand's product with it is 2 lambda (q_j . v).  bf16 path: v's hi
// and lo bf16 parts in two planes, zero-padded to KP.  One thread per row.
__global__ __launch_bounds__(256) void k_prep_u(const float* __restrict__ V, int rows, int rows_pad, int d, int KP,
                                                int mode, int batch, u16* __restrict__ U) {
  const int b = blockIdx.y;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows_pad) return;
  const size_t plane = ((size_t)batch * rows_pad + SLACK) * KP;
  u16* dst = U + ((size_t)b * rows_pad + i) * KP;
  const bool real = i < rows;
  const float* v = V + ((size_t)b * rows + (real ? i : 0)) * d;
  if (mode == MODE_HILO) {
    // (u_h, u_h, u_l) per coordinate against the key rows' (v_h, v_l, v_h)
    for (int k0 = 0; k0 < KP; k0 += 8) {
      u16 w8[8];
      for (int e = 0; e < 8; ++e) {
        const int k = k0 + e, t = k / 3;
        u16 val = 0;
        if (real && t < d) {
          const u16 h = bf16_rne(v[t]);
          val = (k % 3 == 2) ? bf16_rne(v[t] - bf16_f(h)) : h;
        }
        w8[e] = val;
      }
      *reinterpret_cast<u4*>(dst + k0) = pack8(w8);
    }
    return;
  }
  if (mode == MODE_BF16) {
    for (int k = 0; k < KP; k += 2) {
      u16 h[2] = {0, 0}, l[2] = {0, 0};
      for (int e = 0; e < 2; ++e)
        if (real && k + e < d) {
          h[e] = bf16_rne(v[k + e]);
          l[e] = bf16_rne(v[k + e] - bf16_f(h[e]));
        }
      *reinterpret_cast<uint32_t*>(dst + k) = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
      *reinterpret_cast<uint32_t*>(dst + plane + k) = (uint32_t)l[0] | ((uint32_t)l[1] << 16);
    }
    return;
  }
  double vmax = 0.0;
  if (real)
    for (int t = 0; t < d; ++t) vmax = fmax(vmax, fabs((double)v[t]));
  const int qe = grid_exponent(vmax);
  const double q = ldexp(1.0, qe), iq = ldexp(1.0, -qe);
  const int cb = split_corr_begin(d);
  for (int k0 = 0; k0 < KP; k0 += 8) {
    u16 w8[8];
    for (int e = 0; e < 8; ++e) {
      const int k = k0 + e;
      u16 val = 0;
      if (real && k >= 5 && k < 5 + d) {
        val = grid_split((double)v[k - 5], q, iq).g;
      } else if (real && k >= cb && k < cb + 7 * d) {
        const Parts pp = grid_split((double)v[(k - cb) / 7], q, iq);
        const int sl = (k - cb) % 7;
        val = (sl <= 1) ? pp.g : ((sl == 3 || sl == 6) ? pp.r2 : pp.r1);
      }
      w8[e] = val;
    }
    *reinterpret_cast<u4*>(dst + k0) = pack8(w8);
  }
}

// Merge of the row-weighted pass: quad_i = r_i (sum_splits sum_parts pv) /
// (sum_splits s), r_i the row mass, in fp64.  One thread per (problem, row, coordinate).
__global__ __launch_bounds__(256) void k_uw_merge(const float* __restrict__ pv, const float* __restrict__ sp, int ks,
                                                  int batch, MergeRows mr, int d, int ncols, int parts,
                                                  const double* __restrict__ logw, const float* __restrict__ pot,
                                                  const float* __restrict__ lse, double eps,
                                                  double* __restrict__ quad) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)batch * mr.nrows * d) return;
  const int t = (int)(idx % d);
  const int lr = (int)((idx / d) % mr.nrows), b = (int)(idx / ((long long)mr.nrows * d));
  const long long rr = (long long)b * mr.rows + mr.row0 + lr;
  const size_t pr = (size_t)b * mr.prows + lr, pstride = (size_t)batch * mr.prows;
  double S = 0.0, num = 0.0;
#pragma unroll 4
  for (int k = 0; k < ks; ++k) {
    const size_t base = k * pstride + pr;
    for (int part = 0; part < parts; ++part) num += (double)pv[base * ncols + part * d + t];
  }
  for (int k = 0; k < mr.ks_s; ++k) S += (double)sp[k * pstride + pr];
  const double mass = exp(logw[rr] + ((double)pot[rr] - (double)lse[rr]) / eps);
  quad[(size_t)rr * d + t] = mass > 0.0 ? mass * num / S : 0.0;
}

// Centred coordinates of a cloud as an fp32 matrix (rows points per problem).
__global__ __launch_bounds__(256) void k_coords(const void* __restrict__ P, int in_bf16, long long total, int d,
                                                int rows, const double* __restrict__ cen, float* __restrict__ M) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < total) M[i] = (float)ccoord(P, (size_t)(i / d), (int)(i % d), d, in_bf16, cen, (int)(i / ((long long)rows * d)));
}

// HV_i = 2 r v + (2/eps) [ df (r p - PY) + p (P dg) - P(dg q) - 2 (z (r p - PY) - (v.PY) p + quad) ]
// with df = (cr - P dg)/r; G = P [dg, dg q].
__global__ __launch_bounds__(256) void k_hvp_final(const void* __restrict__ P, int in_bf16,
                                                   const float* __restrict__ V, const float* __restrict__ PY,
                                                   const double* __restrict__ mass, const double* __restrict__ zr,
                                                   const double* __restrict__ cr, const float* __restrict__ G,
                                                   const double* __restrict__ quad, long long total, int d,
                                                   int rows, const double* __restrict__ cen, double eps,
                                                   float* __restrict__ out) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const double r = mass[i];
  if (!(r > 0.0)) {
    for (int t = 0; t < d; ++t) out[i * d + t] = 0.f;
    return;
  }
  const float* g = G + i * (d + 1);
  const double df = (cr[i] - (double)g[0]) / r;
  double vpy = 0.0;
  for (int t = 0; t < d; ++t) vpy += (double)V[i * d + t] * (double)PY[i * d + t];
  const double z = zr[i];
  for (int t = 0; t < d; ++t) {
    const double pt = ccoord(P, (size_t)i, t, d, in_bf16, cen, (int)(i / rows));
    const double grad_half = r * pt - (double)PY[i * d + t];
    const double K = 2.0 * (z * grad_half - vpy * pt + quad[i * d + t]);
    const double inner = df * grad_half + pt * (double)g[0] - (double)g[1 + t] - K;
    out[i * d + t] = (float)(2.0 * r * (double)V[i * d + t] + (2.0 / eps) * inner);
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
using LseFn = void (*)(const u16*, const u16*, const float*, const float*, const double*, float*, float2*, int, int,
                       int, int, int, int, float, double, unsigned*, unsigned, unsigned*, NextBias, WvArgs);

template <int MODE, int NCH, int WV>
LseFn lse_fn() {
  // bf16 operands past 256 slots take the K-looped kernel (k_lsek)
  if constexpr ((MODE == MODE_SPLIT && NCH <= MAX_NCH_SPLIT) || (MODE == MODE_BF16 && NCH <= 8))
    return &k_lse<MODE, NCH, 0, WV>;
  else
    return nullptr;
}

template <int MODE, int WV, int... N>
LseFn lse_lookup_impl(int nch, std::integer_sequence<int, N...>) {
  LseFn fn = nullptr;
  ((nch == N + 1 ? (fn = lse_fn<MODE, N + 1, WV>(), 0) : 0), ...);
  return fn;
}

template <int MODE, int WV = 0>
LseFn lse_lookup(int nch) {
  constexpr int MAXN = MODE == MODE_SPLIT ? MAX_NCH_SPLIT : MAX_NCH_BF16;
  return lse_lookup_impl<MODE, WV>(nch, std::make_integer_sequence<int, MAXN>{});
}

sk_status hip_check(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_err("%s: %s", what, hipGetErrorString(e));
    return SK_EHIP;
  }
  return SK_OK;
}

// need: 0 solver, 1 transport and plan products, 2 Hessian-vector products
sk_status check_ws(const sk_problem* p, void* ws, size_t ws_bytes, Layout* L, int need_kind = 0) {
  sk_status st = check_problem(p);
  if (st != SK_OK) return st;
  *L = layout_of(p);
  const size_t need = need_kind == 2 ? L->htotal : (need_kind == 1 ? L->ttotal : L->total);
  if (ws == nullptr || ws_bytes < need) {
    set_err("workspace %s: need %zu bytes, got %zu%s", ws == nullptr ? "is NULL" : "too small", need, ws_bytes,
            need_kind == 2 ? " (HVP calls need sinkhorn_hvp_workspace_bytes)"
                           : (need_kind == 1 ? " (transport calls need sinkhorn_transport_workspace_bytes)" : ""));
    return SK_EWORKSPACE;
  }
  return SK_OK;
}

// Workgroups of `fn` that the current device holds at once (CUs x WGs per CU).
// Cached per (device, kernel) in a fixed table (no heap use, so the
// allocation-free entry point stays allocation-free); a full table just
// queries again.
sk_status resident_capacity(const void* fn, int* out, int block = 256) {
  struct Entry {
    int dev;
    const void* fn;
    int value;
  };
  constexpr int CACHE = 512;
  static std::mutex mu;
  static Entry cache[CACHE];
  static int used = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    set_err("hipGetDevice failed");
    return SK_EHIP;
  }
  std::lock_guard<std::mutex> lock(mu);
  for (int k = 0; k < used; ++k)
    if (cache[k].dev == dev && cache[k].fn == fn) {
      *out = cache[k].value;
      return SK_OK;
    }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, block, 0) != hipSuccess) {
    set_err("occupancy query failed");
    return SK_EHIP;
  }
  *out = std::max(1, cus * std::max(1, per_cu));
  if (used < CACHE) cache[used++] = Entry{dev, fn, *out};
  return SK_OK;
}


// Key operand of one side for the potential pot_in and eps: the split key rows
// (fp32 path) or the half bias (bf16 path).  Returns the key operand and bias.
// Key operand of one side (side 0: keys Y for the f half-step; side 1: keys X)
// for the potential pot_in and eps: the split key rows (fp32 path) or the half
// bias (bf16 path), and the grid quantum of that side (fp32 path).  With
// launch == false nothing is enqueued: the operand's bias was already written
// for this potential and eps by the kernel that produced pot_in.
struct KeyOperand {
  const u16* K = nullptr;
  const float* hb = nullptr;
  const float* qgrid = nullptr;
  unsigned* tag = nullptr;
};

sk_status prep_keys(const sk_problem* p, const void* X, const void* Y, char* w, const Layout& L, const float* pot_in,
                    float eps, int side, hipStream_t stream, KeyOperand* out, bool launch = true) {
  const int B = (int)p->batch;
  const int keys = (int)(side == 0 ? p->m : p->n);
  const int keys_pad = side == 0 ? L.m_pad : L.n_pad;
  const double* knorm = reinterpret_cast<const double*>(w + (side == 0 ? L.yn : L.xn));
  const double* klogw = reinterpret_cast<const double*>(w + (side == 0 ? L.lb : L.la));
  const float* maxabs = reinterpret_cast<const float*>(w + L.maxabs);
  float* qgrid = reinterpret_cast<float*>(w + L.qgrid) + side * B;
  const void* Kraw = side == 0 ? Y : X;
  const float lam = (float)(LOG2E / (double)eps);
  *out = KeyOperand{};
  out->qgrid = qgrid;
  if (L.mode == MODE_SPLIT) {
    u16* kb = reinterpret_cast<u16*>(w + L.kb(side));
    unsigned* tag = reinterpret_cast<unsigned*>(w + L.ktag) + side;
    out->K = kb;
    out->tag = tag;
    if (!launch) return SK_OK;
    // about PREP_SEGS segments per thread when every segment is rebuilt
    const dim3 kgrid((unsigned)(((long long)keys_pad * (L.KP / 8) + 256 * PREP_SEGS - 1) / (256 * PREP_SEGS)), B);
    const double* krn = reinterpret_cast<const double*>(w + (side == 0 ? L.ry : L.rx));
    hipLaunchKernelGGL(k_prep_keys, kgrid, dim3(256), 0, stream, Kraw, L.in_bf16, krn,
                       reinterpret_cast<const double*>(w + L.cen), pot_in, knorm,
                       klogw, keys, keys_pad, (int)p->d, L.KP, lam, eps, maxabs + (side == 0 ? 0 : B),
                       maxabs + (side == 0 ? B : 0), qgrid, tag, kb);
  } else if (L.mode == MODE_HILO) {
    // hi/lo key rows (rebuilt only when lambda changes) and the bias vector lambda*beta
    u16* kb = reinterpret_cast<u16*>(w + L.kb(side));
    unsigned* tag = reinterpret_cast<unsigned*>(w + L.ktag) + side;
    float* hbw = reinterpret_cast<float*>(w + L.hbs(side));
    out->K = kb;
    out->tag = tag;
    out->hb = hbw;
    if (!launch) return SK_OK;
    const long long segs = (long long)keys_pad * (L.KP / 8);
    hipLaunchKernelGGL(k_prep_keys_hilo, dim3((unsigned)((segs + 255) / 256), B), dim3(256), 0, stream, Kraw,
                       L.in_bf16, reinterpret_cast<const double*>(w + L.cen), keys, keys_pad, (int)p->d, L.KP, lam,
                       tag, kb);
    hipLaunchKernelGGL(k_prep_bias, dim3((keys_pad + 255) / 256, B), dim3(256), 0, stream, pot_in, knorm, klogw,
                       keys, keys_pad, eps, lam, hbw);
  } else {
    float* hbw = reinterpret_cast<float*>(w + L.hbs(side));
    out->hb = hbw;
    out->K = reinterpret_cast<const u16*>(w + (side == 0 ? L.qy : L.qx));
    if (!launch) return SK_OK;
    const dim3 pgrid((keys_pad + 255) / 256, B);
    hipLaunchKernelGGL(k_prep_bias, pgrid, dim3(256), 0, stream, pot_in, knorm, klogw, keys, keys_pad, eps, 0.5f,
                       hbw);
  }
  return hip_check("key preparation launch");
}

// The NextBias of a half-step on `side` whose successor runs on 1 - side at
// eps_next (writes the successor's key bias), or an empty one.
NextBias next_bias(const sk_problem* p, char* w, const Layout& L, int side, float eps_next, bool enable) {
  NextBias nb{};
  if (!enable) return nb;
  const int B = (int)p->batch, ns = 1 - side;
  const float* maxabs = reinterpret_cast<const float*>(w + L.maxabs);
  nb.logw = reinterpret_cast<const double*>(w + (side == 0 ? L.la : L.lb));
  nb.qmax = maxabs + (ns == 0 ? 0 : B);
  nb.kmax = maxabs + (ns == 0 ? B : 0);
  nb.lam = (float)(LOG2E / (double)eps_next);
  nb.eps = eps_next;
  nb.rows_pad = side == 0 ? L.n_pad : L.m_pad;
  nb.KP = L.KP;
  nb.cb = split_corr_begin((int)p->d);
  nb.d = (int)p->d;
  if (L.mode == MODE_SPLIT) {
    nb.kb = reinterpret_cast<u16*>(w + L.kb(ns));
  } else {
    nb.hb = reinterpret_cast<float*>(w + L.hbs(ns));
    nb.hscale = L.mode == MODE_HILO ? nb.lam : 0.5f;
  }
  return nb;
}

// Arguments of the K-looped kernel for scores of the query operand Qop (rows
// of one side) against a key operand: the fields every epilogue shares.
KlArgs kl_scores(const Layout& L, const u16* Qop, const KeyOperand& ko, int rows_pad, int keys_pad, int rows,
                 int keys, int B, float lam) {
  KlArgs a{};
  a.A = Qop;
  a.B = ko.K;
  a.hb = ko.hb;
  a.tag = ko.tag;
  a.tag_val = __builtin_bit_cast(unsigned, lam);
  a.a_ld = a.b_ld = L.KP;
  a.a_rows = rows_pad;
  a.b_rows = keys_pad;
  a.a_nkc = a.b_nkc = a.nkc = L.KP / KL_KC;
  a.rows = rows;
  a.keys = keys;
  a.batch = B;
  a.sc = L.mode == MODE_HILO ? 1.f : 2.f * lam;
  a.lam = lam;
  return a;
}

// One half-step.  side 0: f from g (queries X, keys Y); side 1: g from f.
// bias_ready: the key bias for pot_in and eps is already in place (written by
// the producer of pot_in), so no preparation kernel runs.  nb: write the next
// half-step's key bias where the potential is finalised (see NextBias).
sk_status half_step(const sk_problem* p, const void* X, const void* Y, void* ws, const Layout& L,
                    const float* pot_in, float eps, float* pot_out, int side, hipStream_t stream,
                    bool bias_ready = false, NextBias nb = NextBias{}) {
  char* w = static_cast<char*>(ws);
  const int B = (int)p->batch;
  const int rows = (int)(side == 0 ? p->n : p->m);
  const int keys = (int)(side == 0 ? p->m : p->n);
  const int rows_pad = side == 0 ? L.n_pad : L.m_pad;
  const int keys_pad = side == 0 ? L.m_pad : L.n_pad;
  const double* qnorm = reinterpret_cast<const double*>(w + (side == 0 ? L.xn : L.yn));
  const u16* Qop = reinterpret_cast<const u16*>(w + (side == 0 ? L.qx : L.qy));
  const int nch = L.KP / 32;
  const int cfMW = cfg_MW(L.mode, nch), cfR = cfg_R(L.mode, nch), cfTC = cfg_TC(L.mode, nch);
  const float lam = (float)(LOG2E / (double)eps);

  KeyOperand ko;
  sk_status st = prep_keys(p, X, Y, w, L, pot_in, eps, side, stream, &ko, !bias_ready);
  if (st != SK_OK) return st;
  unsigned* status = reinterpret_cast<unsigned*>(w + L.status);
  const double inv_lam = 1.0 / (double)lam;

  if (L.mode == MODE_HILO || (L.mode == MODE_BF16 && p->d > 256)) {
    // K-looped kernel: 256-query x 256-key blocks, splits over key blocks (fp32
    // hi/lo operands; bf16 operands past 256 slots, measured +58% at d = 1024
    // and +1% at d = 512 against 16x16 tiles with the query operand in registers)
    if (L.KP < 2 * KL_KC) {
      set_err("internal: the K-looped half-step needs at least two K chunks (KP = %d)", L.KP);
      return SK_EUNSUPPORTED;
    }
    const int wg_x = (rows + KL_BQ - 1) / KL_BQ;
    const int nblk = (keys + KL_BK - 1) / KL_BK;
    int capacity = 0;
    st = resident_capacity(reinterpret_cast<const void*>(&k_lsek<EPI_LSE>), &capacity, 64 * KL_NW);
    if (st != SK_OK) return st;
    int bps = 0;
    const int ks = choose_key_splits(wg_x * B, nblk, capacity, &bps);
    float2* part = ks > 1 ? reinterpret_cast<float2*>(w + L.part) : nullptr;
    KlArgs ka = kl_scores(L, Qop, ko, rows_pad, keys_pad, rows, keys, B, lam);
    ka.qnorm = qnorm;
    ka.out = pot_out;
    ka.part = part;
    ka.per_split = bps;
    ka.inv_lam = inv_lam;
    ka.status = status;
    ka.nb = ks == 1 ? nb : NextBias{};
    hipLaunchKernelGGL(k_lsek<EPI_LSE>, dim3(wg_x, ks, B), dim3(64 * KL_NW), 0, stream, ka);
    st = hip_check("half-step kernel launch");
    if (st != SK_OK || ks == 1) return st;
    const int total = B * rows;
    hipLaunchKernelGGL(k_merge, dim3((total + 255) / 256), dim3(256), 0, stream, part, ks, total, rows, qnorm,
                       pot_out, inv_lam, status, nb);
    return hip_check("split merge launch");
  }

  LseFn fn = (L.mode == MODE_SPLIT) ? lse_lookup<MODE_SPLIT>(nch) : lse_lookup<MODE_BF16>(nch);
  int tc = cfTC, rq = cfR;
  bool one_split = false;
  if (L.mode == MODE_SPLIT && nch == 1 && (long long)rows * keys <= TINY_WORK) {
    // a tiny problem: one query tile per wave and no key split, so that the
    // half-step is one launch (a split merge would cost as much as the scores)
    fn = &k_lse<MODE_SPLIT, 1, TINY_TC, false, TINY_R>;
    tc = TINY_TC;
    rq = TINY_R;
    one_split = true;
  } else if (L.mode == MODE_SPLIT && nch == 1 && keys < SMALL_KEYS) {
    // fewer keys than a few workgroups' worth of 256-key chunks: 128-key chunks fill the GPU better
    fn = &k_lse<MODE_SPLIT, 1, SMALL_TC>;
    tc = SMALL_TC;
  }
  if (fn == nullptr) {
    set_err("no kernel for %d K chunks", nch);
    return SK_EUNSUPPORTED;
  }
  const int NW = cfg_NW(L.mode, nch);
  const int wg_x = (rows + NW * rq * cfMW - 1) / (NW * rq * cfMW);
  const int CK = tc * cfMW;
  const int total_chunks = (keys + CK - 1) / CK;
  int capacity = 0;
  st = resident_capacity(reinterpret_cast<const void*>(fn), &capacity, 64 * NW);
  if (st != SK_OK) return st;
  int cps = total_chunks;
  const int ks = one_split ? 1 : choose_key_splits(wg_x * B, total_chunks, capacity, &cps);
  float2* part = ks > 1 ? reinterpret_cast<float2*>(w + L.part) : nullptr;
  hipLaunchKernelGGL(fn, dim3(wg_x, ks, B), dim3(64 * NW), 0, stream, Qop, ko.K, ko.hb, ko.qgrid, qnorm, pot_out,
                     part, rows, rows_pad, keys, keys_pad, cps, B, 2.f * lam, inv_lam, ko.tag,
                     __builtin_bit_cast(unsigned, lam), status, ks == 1 ? nb : NextBias{}, WvArgs{});
  st = hip_check("half-step kernel launch");
  if (st != SK_OK || ks == 1) return st;
  const int total = B * rows;
  hipLaunchKernelGGL(k_merge, dim3((total + 255) / 256), dim3(256), 0, stream, part, ks, total, rows, qnorm, pot_out,
                     inv_lam, status, nb);
  return hip_check("split merge launch");
}

using BaryFn = void (*)(const u16*, const u16*, const float*, const u16*, const float*, const double*, const float*,
                        float*, float*, int, int, int, int, int, int, float, float, float*, unsigned*, unsigned,
                        const u16*, float, unsigned*);

template <int MODE, int D>
BaryFn bary_fn_d() {
  constexpr int NCH = MODE == MODE_SPLIT ? split_nch(D) : (D + 31) / 32;
  return &k_bary<MODE, NCH, val_tiles(MODE, D), val_sumcol(MODE, D), true>;
}

template <int MODE, int... N>
BaryFn bary_lookup_impl(int d, std::integer_sequence<int, N...>) {
  BaryFn fn = nullptr;
  ((d == N + 1 ? (fn = bary_fn_d<MODE, N + 1>(), 0) : 0), ...);
  return fn;
}

BaryFn bary_lookup(int mode, int d) {
  if (mode == MODE_SPLIT) return bary_lookup_impl<MODE_SPLIT>(d, std::make_integer_sequence<int, SK_MAX_D_SPLIT>{});
  return bary_lookup_impl<MODE_BF16>(d, std::make_integer_sequence<int, SK_MAX_D_TRANSPORT>{});
}

// Plan pass for wide operands (see EPI_W): per block of L.wt_rows rows of
// `side`, the weights at the rows' fixed offsets (their half-step values lse)
// with their plain sums per split (into bs), times u_ij when the direction
// planes U are given, then their product with the value rows (L.vt, L.ncols
// columns) into the split partials (L.bpv); then `merge` for the block's rows.
template <class Merge>
sk_status wide_pass(const sk_problem* p, const void* X, const void* Y, char* w, const Layout& L, const float* pot_key,
                    const float* lse, float eps, int side, const u16* U, float ugain, hipStream_t stream,
                    const Merge& merge) {
  const int B = (int)p->batch;
  const int rows = (int)(side == 0 ? p->n : p->m);
  const int keys = (int)(side == 0 ? p->m : p->n);
  const int rows_pad = side == 0 ? L.n_pad : L.m_pad;
  const int keys_pad = side == 0 ? L.m_pad : L.n_pad;
  const double* qnorm = reinterpret_cast<const double*>(w + (side == 0 ? L.xn : L.yn));
  const u16* Qop = reinterpret_cast<const u16*>(w + (side == 0 ? L.qx : L.qy));
  KeyOperand ko;
  sk_status st = prep_keys(p, X, Y, w, L, pot_key, eps, side, stream, &ko);
  if (st != SK_OK) return st;
  if (L.KP < 2 * KL_KC || L.ncols % KL_BK != 0) {
    set_err("internal: wide plan pass with KP = %d, %d value columns", L.KP, L.ncols);
    return SK_EUNSUPPORTED;
  }
  const int nblk = (keys + KL_BK - 1) / KL_BK, kcov = nblk * KL_BK;
  const int rb = L.wt_rows;
  const int wg_full = (std::min(rb, rows) + KL_BQ - 1) / KL_BQ;
  const float lam = (float)(LOG2E / (double)eps);
  const int planes = L.mode == MODE_BF16 ? 2 : 1;  // direction planes (hi, lo) of the bf16 path
  int cap_w = 0, cap_g = 0;
  st = resident_capacity(reinterpret_cast<const void*>(&k_lsek<EPI_W>), &cap_w, 64 * KL_NW);
  if (st == SK_OK) st = resident_capacity(reinterpret_cast<const void*>(&k_lsek<EPI_GEMM>), &cap_g, 64 * KL_NW);
  if (st != SK_OK) return st;
  // splits of the weights pass over key blocks and of the product over its K
  // range (hi keys, then lo keys); the partials of one row block hold 16 splits
  const int ncolt = L.ncols / KL_BK, total_kc = 2 * kcov / KL_KC;
  int cps = 0, bps_w = 0;
  const int ks = choose_key_splits(wg_full * ncolt * B, total_kc, cap_g, &cps, 16);
  const int ks_w = choose_key_splits(wg_full * B, nblk, cap_w, &bps_w, 16);
  u16* wt = reinterpret_cast<u16*>(w + L.wt);
  float* sp = reinterpret_cast<float*>(w + L.bs);
  unsigned* status = reinterpret_cast<unsigned*>(w + L.status);
  for (int r0 = 0; r0 < rows; r0 += rb) {
    const int nrows = std::min(rb, rows - r0);
    const int wg = (nrows + KL_BQ - 1) / KL_BQ;
    KlArgs aw = kl_scores(L, Qop, ko, rows_pad, keys_pad, rows, keys, B, lam);
    aw.a_row0 = aw.row0 = r0;
    aw.qnorm = qnorm;
    aw.lse = lse;
    aw.wt = wt;
    aw.wt_ld = 2 * kcov;
    aw.kcov = kcov;
    aw.wt_rows = rb;
    aw.prows = rb;
    aw.sp = sp;
    aw.per_split = bps_w;
    aw.status = status;
    hipLaunchKernelGGL(k_lsek<EPI_W>, dim3(wg, ks_w, B), dim3(64 * KL_NW), 0, stream, aw);
    if (U != nullptr) {
      KlArgs au = aw;
      au.A = U;
      au.hb = nullptr;
      au.tag = nullptr;
      au.sp = nullptr;
      au.a_plane = ((long long)B * rows_pad + SLACK) * L.KP;
      au.nkc = planes * (L.KP / KL_KC);
      au.ugain = ugain;
      hipLaunchKernelGGL(k_lsek<EPI_U>, dim3(wg, ks_w, B), dim3(64 * KL_NW), 0, stream, au);
    }
    KlArgs ag{};
    ag.A = wt;
    ag.B = reinterpret_cast<const u16*>(w + L.vt);
    ag.a_ld = 2 * kcov;
    ag.a_rows = rb;
    ag.a_nkc = total_kc;
    ag.b_ld = kcov;
    ag.b_rows = L.ncols;
    ag.b_nkc = kcov / KL_KC;
    ag.rows = rows;
    ag.row0 = r0;
    ag.prows = rb;
    ag.per_split = cps;
    ag.total_kc = total_kc;
    ag.ncolt = ncolt;
    ag.nc = L.ncols;
    ag.pv = reinterpret_cast<float*>(w + L.bpv);
    ag.batch = B;
    hipLaunchKernelGGL(k_lsek<EPI_GEMM>, dim3(wg, ncolt * ks, B), dim3(64 * KL_NW), 0, stream, ag);
    st = hip_check("wide plan pass launch");
    if (st == SK_OK) st = merge(MergeRows{rows, r0, nrows, rb, ks_w}, ks);
    if (st != SK_OK) return st;
  }
  return SK_OK;
}

// Value rows of a wide pass (k_prep_vt) for the keys of `side`.
sk_status wide_values(const sk_problem* p, const void* Kraw, char* w, const Layout& L, int side, const float* M,
                      int c, int col0, int cb, hipStream_t stream) {
  const int B = (int)p->batch, d = (int)p->d;
  const int keys = (int)(side == 0 ? p->m : p->n);
  const int kcov = (keys + KL_BK - 1) / KL_BK * KL_BK;
  const long long nvec = (long long)L.ncols * (kcov / 8);
  hipLaunchKernelGGL(k_prep_vt, dim3((unsigned)((nvec + 255) / 256), B), dim3(256), 0, stream, Kraw, L.in_bf16,
                     reinterpret_cast<const double*>(w + L.cen), M, c, col0, cb, val_parts(L.mode), keys, kcov, d,
                     L.ncols, reinterpret_cast<u16*>(w + L.vt));
  return hip_check("value rows launch");
}

// Barycentric projection (and gradient) of the rows of one side: side 0 the
// points of X against Y, side 1 the points of Y against X.
sk_status transport(const sk_problem* p, const void* X, const void* Y, void* ws, const Layout& L, const float* f,
                    const float* g, float eps, float* bary, float* grad, int side, hipStream_t stream) {
  char* w = static_cast<char*>(ws);
  const int B = (int)p->batch, d = (int)p->d;
  const int rows = (int)(side == 0 ? p->n : p->m);
  const int keys = (int)(side == 0 ? p->m : p->n);
  const int rows_pad = side == 0 ? L.n_pad : L.m_pad;
  const int keys_pad = side == 0 ? L.m_pad : L.n_pad;
  const double* qnorm = reinterpret_cast<const double*>(w + (side == 0 ? L.xn : L.yn));
  const double* qlogw = reinterpret_cast<const double*>(w + (side == 0 ? L.la : L.lb));
  const u16* Qop = reinterpret_cast<const u16*>(w + (side == 0 ? L.qx : L.qy));
  const void* Praw = side == 0 ? X : Y;
  const void* Kraw = side == 0 ? Y : X;
  const float* pot_row = side == 0 ? f : g;
  float* lse = reinterpret_cast<float*>(w + L.scratch);

  if (L.wide) {
    // the rows' half-step values fix their offsets; then the weights pass with
    // the coordinates (and a ones column for the weight sums) as values
    sk_status st = half_step(p, X, Y, ws, L, side == 0 ? g : f, eps, lse, side, stream);
    if (st == SK_OK) st = wide_values(p, Kraw, w, L, side, nullptr, 0, 0, 0, stream);
    if (st != SK_OK) return st;
    const float lam = (float)(LOG2E / (double)eps);
    return wide_pass(p, X, Y, w, L, side == 0 ? g : f, lse, eps, side, nullptr, 1.f, stream,
                     [&](const MergeRows& mr, int ks) {
                       const long long total = (long long)B * mr.nrows * d;
                       hipLaunchKernelGGL(k_bary_merge, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                                          reinterpret_cast<const float*>(w + L.bpv),
                                          reinterpret_cast<const float*>(w + L.bs), ks, B, mr, d, L.ncols,
                                          val_parts(L.mode), Praw, L.in_bf16, pot_row, lse, qlogw, (double)eps,
                                          nullptr, qnorm, 1.0 / (double)lam,
                                          reinterpret_cast<const double*>(w + L.cen), nullptr, bary, grad);
                       return hip_check("transport merge launch");
                     });
  }

  // 1. The key operand of this side for the other potential and eps.  The P.V
  //    pass keeps lazy row offsets, so no half-step runs first: its merge
  //    recovers each row's log-sum-exp (into scratch) from the offsets and sums.
  KeyOperand ko;
  sk_status st = prep_keys(p, X, Y, w, L, side == 0 ? g : f, eps, side, stream, &ko);
  if (st != SK_OK) return st;

  // 2. Value operand from the other cloud's coordinates.
  u16* vt = reinterpret_cast<u16*>(w + L.vt);
  const int nc = val_tiles(L.mode, d) * 16;
  const long long nvec = (long long)(keys_pad / VK) * nc * (VK / 8);
  const int sumcol = val_sumcol(L.mode, d) ? 1 : 0;
  const double* krn = reinterpret_cast<const double*>(w + (side == 0 ? L.ry : L.rx));
  const double* cen = reinterpret_cast<const double*>(w + L.cen);
  unsigned* status = reinterpret_cast<unsigned*>(w + L.status);
  // bf16 inputs: fp16 values and weights (the P.V pass's HALF path), scaled by the key cloud's extent
  const float* half_max =
      L.mode == MODE_BF16 ? reinterpret_cast<const float*>(w + L.maxabs) + (side == 0 ? B : 0) : nullptr;
  hipLaunchKernelGGL(k_prep_vals, dim3((unsigned)((nvec + 255) / 256), B), dim3(256), 0, stream, Kraw, L.mode,
                     L.in_bf16, krn, cen, keys, keys_pad, d, nc, sumcol, half_max, vt);
  st = hip_check("value preparation launch");
  if (st != SK_OK) return st;

  // 3. The P.V pass, split over keys when rows alone do not fill the GPU.
  BaryFn fn = bary_lookup(L.mode, d);
  if (fn == nullptr) {
    set_err("no transport kernel for d = %d", d);
    return SK_EUNSUPPORTED;
  }
  const int nch = L.KP / 32;
  const int R = bary_R(nch, val_tiles(L.mode, d)), NWb = bary_NW(L.mode, nch, val_tiles(L.mode, d), 0);
  const int wg_x = (rows + NWb * R * 16 - 1) / (NWb * R * 16);
  const int CKb = bary_TCB(nch, val_tiles(L.mode, d)) * VK;
  const int total_chunks = (keys + CKb - 1) / CKb;
  int capacity = 0;
  st = resident_capacity(reinterpret_cast<const void*>(fn), &capacity, 64 * NWb);
  if (st != SK_OK) return st;
  int cps = 0;
  const int ks_cap = (int)std::min<size_t>(16, std::max<size_t>(1, L.bpv_bytes / (4 * (size_t)B * rows * nc)));
  const int ks = choose_key_splits(wg_x * B, total_chunks, capacity, &cps, ks_cap);
  float* bpv = reinterpret_cast<float*>(w + L.bpv);
  float* bs = reinterpret_cast<float*>(w + L.bs);
  float* bm = reinterpret_cast<float*>(w + L.bm);
  const float lam = (float)(LOG2E / (double)eps);
  hipLaunchKernelGGL(fn, dim3(wg_x, ks, B), dim3(64 * NWb), 0, stream, Qop, ko.K, ko.hb, vt, ko.qgrid, qnorm, nullptr,
                     bpv, bs, rows, rows_pad, keys, keys_pad, cps, B, lam, 2.f * lam, bm, ko.tag,
                     __builtin_bit_cast(unsigned, lam), nullptr, 1.f, status);
  st = hip_check("transport kernel launch");
  if (st != SK_OK) return st;

  // 4. Merge the splits, divide, form the gradient.
  const long long total = (long long)B * rows * d;
  const MergeRows mr{rows, 0, rows, rows, sumcol ? 0 : ks};
  hipLaunchKernelGGL(k_bary_merge, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, bpv, bs, ks, B, mr,
                     d, nc, val_parts(L.mode), Praw, L.in_bf16, pot_row, lse, qlogw, (double)eps, bm, qnorm,
                     1.0 / (double)lam, cen, half_max, bary, L.cosine ? nullptr : grad);
  st = hip_check("transport merge launch");
  if (st != SK_OK || !L.cosine || grad == nullptr) return st;
  const double* qrn = reinterpret_cast<const double*>(w + (side == 0 ? L.rx : L.ry));
  const long long nrows = (long long)B * rows;
  hipLaunchKernelGGL(k_cosine_grad, dim3((unsigned)((nrows + 255) / 256)), dim3(256), 0, stream, bary, Praw,
                     L.in_bf16, qrn, pot_row, lse, qlogw, (double)eps, nrows, d, grad);
  return hip_check("cosine gradient launch");
}

// ---------------------------------------------------------------------------
// Plan application (vector- and matrix-transport products) and HVP drivers
// ---------------------------------------------------------------------------
template <int MODE, int D>
BaryFn apply_fn_d(int nct) {
  constexpr int NCH = MODE == MODE_SPLIT ? split_nch(D) : (D + 31) / 32;
  if (nct == 1) return &k_bary<MODE, NCH, 1, true>;
  if (nct == 4) return &k_bary<MODE, NCH, 4, true>;
  return &k_bary<MODE, NCH, 13, true>;
}

template <int MODE, int... N>
BaryFn apply_lookup_impl(int d, int nct, std::integer_sequence<int, N...>) {
  BaryFn fn = nullptr;
  ((d == N + 1 ? (fn = apply_fn_d<MODE, N + 1>(nct), 0) : 0), ...);
  return fn;
}

BaryFn apply_lookup(int mode, int d, int nct) {
  if (mode == MODE_SPLIT)
    return apply_lookup_impl<MODE_SPLIT>(d, nct, std::make_integer_sequence<int, SK_MAX_D_SPLIT>{});
  return apply_lookup_impl<MODE_BF16>(d, nct, std::make_integer_sequence<int, SK_MAX_D_TRANSPORT>{});
}

// out[b][row][k] = sum_j P_ij M[b][j][k] (k < c) for one side (side 0: rows are
// the points of X, keys those of Y), at potentials pot_row / pot_key whose
// half-step values for the rows are lse.  Columns go in passes of APPLY_COLS.
unsigned blocks_for(long long n) { return (unsigned)((n + 255) / 256); }

// wmode (one column only): 0 plain; 1 also store the rows' mass / weight sum in
// wscale; 2 reuse wscale and skip the weight sums (same potentials, offsets and
// side as the call that stored it).
sk_status apply_plan(const sk_problem* p, const void* X, const void* Y, char* w, const Layout& L,
                     const float* pot_row, const float* pot_key, const float* lse, float eps, int side,
                     const float* M, int c, float* out, hipStream_t stream, int wmode = 0,
                     double* wscale = nullptr) {
  const int B = (int)p->batch, d = (int)p->d;
  const int rows = (int)(side == 0 ? p->n : p->m);
  const int keys = (int)(side == 0 ? p->m : p->n);
  const int rows_pad = side == 0 ? L.n_pad : L.m_pad;
  const int keys_pad = side == 0 ? L.m_pad : L.n_pad;
  const double* qnorm = reinterpret_cast<const double*>(w + (side == 0 ? L.xn : L.yn));
  const double* qlogw = reinterpret_cast<const double*>(w + (side == 0 ? L.la : L.lb));
  const u16* Qop = reinterpret_cast<const u16*>(w + (side == 0 ? L.qx : L.qy));
  if (L.wide) {
    for (int col0 = 0; col0 < c; col0 += L.wide_cols) {
      const int cb = std::min(L.wide_cols, c - col0);
      sk_status st = wide_values(p, side == 0 ? Y : X, w, L, side, M, c, col0, cb, stream);
      if (st == SK_OK)
        st = wide_pass(p, X, Y, w, L, pot_key, lse, eps, side, nullptr, 1.f, stream,
                       [&](const MergeRows& mr, int ks) {
                         const long long total = (long long)B * mr.nrows * cb;
                         hipLaunchKernelGGL(k_apply_merge, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                                            stream, reinterpret_cast<const float*>(w + L.bpv),
                                            reinterpret_cast<const float*>(w + L.bs), ks, B, mr, cb, L.ncols, c, col0,
                                            qlogw, pot_row, lse, (double)eps, out);
                         return hip_check("plan-application merge launch");
                       });
      if (st != SK_OK) return st;
    }
    return SK_OK;
  }
  KeyOperand ko;
  sk_status st = prep_keys(p, X, Y, w, L, pot_key, eps, side, stream, &ko);
  if (st != SK_OK) return st;
  u16* vt = reinterpret_cast<u16*>(w + L.vt);
  float* bpv = reinterpret_cast<float*>(w + L.bpv);
  float* bs = reinterpret_cast<float*>(w + L.bs);
  const float lam = (float)(LOG2E / (double)eps);
  const int nch = L.KP / 32;
  if (c == 1) {
    // one vector (each conjugate-gradient product of the HVP): the half-step
    // kernel sums w_j 2^(s - M_i) beside the weights, one FMA per score, in
    // place of the hi/lo bf16 product with a 16-column value tile
    // the launch shape comes from the kernel with sums in both cases, so that the
    // passes of one side split their keys alike and sum in the same order
    const bool sums = wmode != 2;
    LseFn fn1 = (L.mode == MODE_SPLIT) ? lse_lookup<MODE_SPLIT, 1>(nch) : lse_lookup<MODE_BF16, 1>(nch);
    LseFn fn2 = (L.mode == MODE_SPLIT) ? lse_lookup<MODE_SPLIT, 2>(nch) : lse_lookup<MODE_BF16, 2>(nch);
    int tc = cfg_TC(L.mode, nch);
    if (L.mode == MODE_SPLIT && nch == 1 && keys < SMALL_KEYS) {
      fn1 = &k_lse<MODE_SPLIT, 1, SMALL_TC, 1>;
      fn2 = &k_lse<MODE_SPLIT, 1, SMALL_TC, 2>;
      tc = SMALL_TC;
    }
    LseFn fn = sums ? fn1 : fn2;
    if (fn == nullptr) {
      set_err("no plan-product kernel for %d K chunks", nch);
      return SK_EUNSUPPORTED;
    }
    const int NW = cfg_NW(L.mode, nch), MW = cfg_MW(L.mode, nch);
    const int wg_x = (rows + NW * cfg_R(L.mode, nch) * MW - 1) / (NW * cfg_R(L.mode, nch) * MW);
    const int total_chunks = (keys + tc * MW - 1) / (tc * MW);
    int capacity = 0;
    st = resident_capacity(reinterpret_cast<const void*>(fn1), &capacity, 64 * NW);
    if (st != SK_OK) return st;
    int cps = 0;
    const int ks = choose_key_splits(wg_x * B, total_chunks, capacity, &cps);
    float2* part = reinterpret_cast<float2*>(w + L.part);
    hipLaunchKernelGGL(fn, dim3(wg_x, ks, B), dim3(64 * NW), 0, stream, Qop, ko.K, ko.hb, ko.qgrid, qnorm, nullptr,
                       part, rows, rows_pad, keys, keys_pad, cps, B, 2.f * lam, 1.0 / (double)lam, ko.tag,
                       __builtin_bit_cast(unsigned, lam), reinterpret_cast<unsigned*>(w + L.status), NextBias{},
                       WvArgs{M, lse});
    st = hip_check("plan-product kernel launch");
    if (st != SK_OK) return st;
    hipLaunchKernelGGL(k_wv_merge, dim3(blocks_for((long long)B * rows)), dim3(256), 0, stream, part, ks, B, rows,
                       qlogw, pot_row, lse, (double)eps, wscale != nullptr ? wmode : 0, wscale, out);
    return hip_check("plan-product merge launch");
  }
  for (int col0 = 0; col0 < c; col0 += APPLY_COLS) {
    const int cb = std::min(APPLY_COLS, c - col0);
    const int nct = apply_tiles(cb), nc = nct * 16;
    const int R = bary_R(nch, nct);
    const int CKb = bary_TCB(nch, nct) * VK;
    const int total_chunks = (keys + CKb - 1) / CKb;
    const int NWb = bary_NW(L.mode, nch, nct, 0);
    const int wg_x = (rows + NWb * R * 16 - 1) / (NWb * R * 16);
    const long long nvec = (long long)(keys_pad / VK) * nc * (VK / 8);
    hipLaunchKernelGGL(k_prep_mat, dim3((unsigned)((nvec + 255) / 256), B), dim3(256), 0, stream, M, keys, keys_pad,
                       c, col0, cb, nc, vt);
    st = hip_check("matrix preparation launch");
    if (st != SK_OK) return st;
    BaryFn fn = apply_lookup(L.mode, d, nct);
    if (fn == nullptr) {
      set_err("no plan-application kernel for d = %d", d);
      return SK_EUNSUPPORTED;
    }
    int capacity = 0;
    st = resident_capacity(reinterpret_cast<const void*>(fn), &capacity, 64 * NWb);
    if (st != SK_OK) return st;
    const int ks_cap = (int)std::min<size_t>(16, std::max<size_t>(1, L.bpv_bytes / (4 * (size_t)B * rows * nc)));
    int cps = 0;
    const int ks = choose_key_splits(wg_x * B, total_chunks, capacity, &cps, ks_cap);
    hipLaunchKernelGGL(fn, dim3(wg_x, ks, B), dim3(64 * NWb), 0, stream, Qop, ko.K, ko.hb, vt, ko.qgrid, qnorm, lse,
                       bpv, bs, rows, rows_pad, keys, keys_pad, cps, B, lam, 2.f * lam, nullptr, ko.tag,
                       __builtin_bit_cast(unsigned, lam), nullptr, 1.f, reinterpret_cast<unsigned*>(w + L.status));
    st = hip_check("plan-application kernel launch");
    if (st != SK_OK) return st;
    const long long total = (long long)B * rows * cb;
    const MergeRows mr{rows, 0, rows, rows, 0};
    hipLaunchKernelGGL(k_apply_merge, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, bpv, nullptr, ks,
                       B, mr, cb, nc, c, col0, qlogw, pot_row, lse, (double)eps, out);
    st = hip_check("plan-application merge launch");
    if (st != SK_OK) return st;
  }
  return SK_OK;
}

// Row-weighted plan pass kernels: weights P_ij (q_j . v_i) applied to the
// fixed cloud's coordinates (no ones column; the weight sums come from the VALU).
template <int MODE, int D>
BaryFn uw_fn_d() {
  constexpr int NCH = MODE == MODE_SPLIT ? split_nch(D) : (D + 31) / 32;
  return &k_bary<MODE, NCH, val_tiles(MODE, D), false, false, MODE == MODE_SPLIT ? 1 : 2>;
}
template <int MODE, int... N>
BaryFn uw_lookup_impl(int d, std::integer_sequence<int, N...>) {
  BaryFn fn = nullptr;
  ((d == N + 1 ? (fn = uw_fn_d<MODE, N + 1>(), 0) : 0), ...);
  return fn;
}
BaryFn uw_lookup(int mode, int d) {
  if (mode == MODE_SPLIT) return uw_lookup_impl<MODE_SPLIT>(d, std::make_integer_sequence<int, SK_MAX_D_SPLIT>{});
  return uw_lookup_impl<MODE_BF16>(d, std::make_integer_sequence<int, SK_MAX_D_TRANSPORT>{});
}

// quad_i = sum_j P_ij (q_j . v_i) q_j = M_i v_i with M_i = sum_j P_ij q_j q_j^T, for
// the rows of `side` (q the other cloud), in one streaming pass: the direction v
// enters as a second query operand whose contraction with the key rows gives
// q_j . v_i beside each score.  quad is [B][rows][d] fp64.
sk_status apply_uw(const sk_problem* p, const void* X, const void* Y, char* w, const Layout& L, const float* pot_row,
                   const float* pot_key, const float* lse, float eps, int side, const float* Vdir, double* quad,
                   hipStream_t stream) {
  const int B = (int)p->batch, d = (int)p->d;
  const int rows = (int)(side == 0 ? p->n : p->m);
  const int keys = (int)(side == 0 ? p->m : p->n);
  const int rows_pad = side == 0 ? L.n_pad : L.m_pad;
  const int keys_pad = side == 0 ? L.m_pad : L.n_pad;
  const double* qnorm = reinterpret_cast<const double*>(w + (side == 0 ? L.xn : L.yn));
  const double* qlogw = reinterpret_cast<const double*>(w + (side == 0 ? L.la : L.lb));
  const u16* Qop = reinterpret_cast<const u16*>(w + (side == 0 ? L.qx : L.qy));
  const void* Kraw = side == 0 ? Y : X;
  u16* U = reinterpret_cast<u16*>(w + L.h_u);
  if (L.wide) {
    hipLaunchKernelGGL(k_prep_u, dim3((rows_pad + 255) / 256, B), dim3(256), 0, stream, Vdir, rows, rows_pad, d,
                       L.KP, L.mode, B, U);
    sk_status st = wide_values(p, Kraw, w, L, side, nullptr, 0, 0, 0, stream);
    if (st != SK_OK) return st;
    // the hi/lo key rows hold 2 lambda (y - c)
    const float ugain = L.mode == MODE_HILO ? (float)((double)eps / (2.0 * LOG2E)) : 1.f;
    return wide_pass(p, X, Y, w, L, pot_key, lse, eps, side, U, ugain, stream, [&](const MergeRows& mr, int ks) {
      const long long total = (long long)B * mr.nrows * d;
      hipLaunchKernelGGL(k_uw_merge, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                         reinterpret_cast<const float*>(w + L.bpv), reinterpret_cast<const float*>(w + L.bs), ks, B,
                         mr, d, L.ncols, val_parts(L.mode), qlogw, pot_row, lse, (double)eps, quad);
      return hip_check("row-weighted merge launch");
    });
  }
  KeyOperand ko;
  sk_status st = prep_keys(p, X, Y, w, L, pot_key, eps, side, stream, &ko);
  if (st != SK_OK) return st;
  hipLaunchKernelGGL(k_prep_u, dim3((rows_pad + 255) / 256, B), dim3(256), 0, stream, Vdir, rows, rows_pad, d, L.KP,
                     L.mode, B, U);
  u16* vt = reinterpret_cast<u16*>(w + L.vt);
  const int nct = val_tiles(L.mode, d), nc = nct * 16;
  const long long nvec = (long long)(keys_pad / VK) * nc * (VK / 8);
  const double* krn = reinterpret_cast<const double*>(w + (side == 0 ? L.ry : L.rx));
  hipLaunchKernelGGL(k_prep_vals, dim3((unsigned)((nvec + 255) / 256), B), dim3(256), 0, stream, Kraw, L.mode,
                     L.in_bf16, krn, reinterpret_cast<const double*>(w + L.cen), keys, keys_pad, d, nc, 0, nullptr, vt);
  st = hip_check("direction and value preparation launch");
  if (st != SK_OK) return st;
  BaryFn fn = uw_lookup(L.mode, d);
  if (fn == nullptr) {
    set_err("no row-weighted plan kernel for d = %d", d);
    return SK_EUNSUPPORTED;
  }
  const int nch = L.KP / 32;
  const int R = bary_R(nch, nct), NWb = bary_NW(L.mode, nch, nct, L.mode == MODE_SPLIT ? 1 : 2);
  const int CKb = bary_TCB(nch, nct) * VK;
  const int total_chunks = (keys + CKb - 1) / CKb;
  const int wg_x = (rows + NWb * R * 16 - 1) / (NWb * R * 16);
  int capacity = 0;
  st = resident_capacity(reinterpret_cast<const void*>(fn), &capacity, 64 * NWb);
  if (st != SK_OK) return st;
  const int ks_cap = (int)std::min<size_t>(16, std::max<size_t>(1, L.bpv_bytes / (4 * (size_t)B * rows * nc)));
  int cps = 0;
  const int ks = choose_key_splits(wg_x * B, total_chunks, capacity, &cps, ks_cap);
  float* bpv = reinterpret_cast<float*>(w + L.bpv);
  float* bs = reinterpret_cast<float*>(w + L.bs);
  const float lam = (float)(LOG2E / (double)eps);
  // the fp32 key operand holds 2 lambda q
  const float ugain = L.mode == MODE_SPLIT ? 1.f / (2.f * lam) : 1.f;
  hipLaunchKernelGGL(fn, dim3(wg_x, ks, B), dim3(64 * NWb), 0, stream, Qop, ko.K, ko.hb, vt, ko.qgrid, qnorm, lse, bpv,
                     bs, rows, rows_pad, keys, keys_pad, cps, B, lam, 2.f * lam, nullptr, ko.tag,
                     __builtin_bit_cast(unsigned, lam), U, ugain, reinterpret_cast<unsigned*>(w + L.status));
  st = hip_check("row-weighted plan kernel launch");
  if (st != SK_OK) return st;
  const long long total = (long long)B * rows * d;
  const MergeRows mr{rows, 0, rows, rows, ks};
  hipLaunchKernelGGL(k_uw_merge, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, bpv, bs, ks, B, mr, d,
                     nc, val_parts(L.mode), qlogw, pot_row, lse, (double)eps, quad);
  return hip_check("row-weighted merge launch");
}


// Hessian of the entropic OT value in the points of one cloud (side 0: X,
// side 1: Y) applied to V, at potentials (f, g) taken as optimal.  Moving the
// points along V changes the costs by dC and the potentials by (df, dg) that
// keep the plan's marginals; eliminating df leaves the Schur system in dg,
// solved by conjugate gradients whose products are plan applications.
sk_status hvp(const sk_problem* p, const void* X, const void* Y, char* w, const Layout& L, const float* f,
              const float* g, float eps, const float* V, int64_t cg_iters, float cg_tol, float* out, int side,
              hipStream_t s) {
  const int B = (int)p->batch, d = (int)p->d;
  const int rows = (int)(side == 0 ? p->n : p->m);
  const int keys = (int)(side == 0 ? p->m : p->n);
  const void* Praw = side == 0 ? X : Y;
  const void* Qraw = side == 0 ? Y : X;
  const float* pot_r = side == 0 ? f : g;
  const float* pot_k = side == 0 ? g : f;
  const double* logw_r = reinterpret_cast<const double*>(w + (side == 0 ? L.la : L.lb));
  const double* logw_k = reinterpret_cast<const double*>(w + (side == 0 ? L.lb : L.la));
  float* lse_r = reinterpret_cast<float*>(w + L.h_lse_r);
  float* lse_k = reinterpret_cast<float*>(w + L.h_lse_k);
  double* mr = reinterpret_cast<double*>(w + L.h_mr);
  double* mk = reinterpret_cast<double*>(w + L.h_mk);
  float* py = reinterpret_cast<float*>(w + L.h_py);
  float* mat = reinterpret_cast<float*>(w + L.h_mat);
  float* wk = reinterpret_cast<float*>(w + L.h_w);
  float* gm = reinterpret_cast<float*>(w + L.h_g);
  double* quad = reinterpret_cast<double*>(w + L.h_quad);
  double* zr = reinterpret_cast<double*>(w + L.h_zr);
  double* cr = reinterpret_cast<double*>(w + L.h_cr);
  double* rhs = reinterpret_cast<double*>(w + L.h_rhs);
  double* dg = reinterpret_cast<double*>(w + L.h_dg);
  double* res = reinterpret_cast<double*>(w + L.h_res);
  double* pd = reinterpret_cast<double*>(w + L.h_pd);
  float* pdf = reinterpret_cast<float*>(w + L.h_pdf);
  float* tv = reinterpret_cast<float*>(w + L.h_t);
  float* qv = reinterpret_cast<float*>(w + L.h_q);
  double* stt = reinterpret_cast<double*>(w + L.h_st);
  const long long nr = (long long)B * rows, nk = (long long)B * keys;
  const int in16 = L.in_bf16;
  void* vw = static_cast<void*>(w);

  // 1. both sides' row log-sum-exps (fixed offsets of every plan pass) and masses
  sk_status st = half_step(p, X, Y, vw, L, pot_k, eps, lse_r, side, s);
  if (st == SK_OK) st = half_step(p, X, Y, vw, L, pot_r, eps, lse_k, 1 - side, s);
  if (st != SK_OK) return st;
  hipLaunchKernelGGL(k_mass, dim3(blocks_for(nr)), dim3(256), 0, s, logw_r, pot_r, lse_r, (double)eps, nr, mr);
  hipLaunchKernelGGL(k_mass, dim3(blocks_for(nk)), dim3(256), 0, s, logw_k, pot_k, lse_k, (double)eps, nk, mk);
  // 2. P Q (the plan applied to the fixed cloud's coordinates)
  const double* cen = reinterpret_cast<const double*>(w + L.cen);
  hipLaunchKernelGGL(k_coords, dim3(blocks_for(nk * d)), dim3(256), 0, s, Qraw, in16, nk * d, d, keys, cen, mat);
  st = hip_check("HVP set-up launch");
  if (st == SK_OK) st = apply_plan(p, X, Y, w, L, pot_r, pot_k, lse_r, eps, side, mat, d, py, s);
  if (st != SK_OK) return st;
  // 3. right-hand side: cr per moving row, then P^T [z, v, cr/r] per fixed row
  hipLaunchKernelGGL(k_hvp_rows, dim3(blocks_for(nr)), dim3(256), 0, s, Praw, in16, V, py, mr, nr, d, rows, cen, zr, cr,
                     mat);
  st = hip_check("HVP rows launch");
  if (st == SK_OK) st = apply_plan(p, X, Y, w, L, pot_k, pot_r, lse_k, eps, 1 - side, mat, d + 2, wk, s);
  if (st != SK_OK) return st;
  hipLaunchKernelGGL(k_hvp_rhs, dim3(blocks_for(nk)), dim3(256), 0, s, Qraw, in16, wk, nk, d, keys, cen, rhs);
  // 4. conjugate gradients on the Schur system in dg
  const int nblk = (keys + CG_BLK - 1) / CG_BLK;
  double* pa = reinterpret_cast<double*>(w + L.h_part);
  double* pb = pa + (size_t)B * nblk;
  double* st_a = stt;
  double* st_b = stt + 4 * (size_t)B;
  const dim3 vgrid(nblk, B);
  hipLaunchKernelGGL(k_cg_init1, vgrid, dim3(256), 0, s, rhs, keys, nblk, res, pa);
  hipLaunchKernelGGL(k_cg_init2, vgrid, dim3(256), 0, s, mk, keys, nblk, pa, dg, res, pd, pdf, pb);
  hipLaunchKernelGGL(k_cg_init3, dim3(B), dim3(256), 0, s, nblk, pb, st_a);
  st = hip_check("CG set-up launch");
  if (st != SK_OK) return st;
  const double tol2 = (double)cg_tol * (double)cg_tol;
  // the plan passes' weight sums depend on the potentials and offsets only: the
  // first iteration stores mass / sum per row and side, later ones reuse it
  double* wsr = reinterpret_cast<double*>(w + L.h_wsr);
  double* wsk = reinterpret_cast<double*>(w + L.h_wsk);
  for (int64_t it = 0; it < cg_iters; ++it) {
    const int wm = it == 0 ? 1 : 2;
    st = apply_plan(p, X, Y, w, L, pot_r, pot_k, lse_r, eps, side, pdf, 1, tv, s, wm, wsr);
    if (st != SK_OK) return st;
    hipLaunchKernelGGL(k_div_mass, dim3(blocks_for(nr)), dim3(256), 0, s, tv, mr, nr);
    st = apply_plan(p, X, Y, w, L, pot_k, pot_r, lse_k, eps, 1 - side, tv, 1, qv, s, wm, wsk);
    if (st != SK_OK) return st;
    double* st_in = (it % 2 == 0) ? st_a : st_b;
    double* st_out = (it % 2 == 0) ? st_b : st_a;
    hipLaunchKernelGGL(k_cg_a, vgrid, dim3(256), 0, s, qv, mk, keys, nblk, pd, pa);
    hipLaunchKernelGGL(k_cg_b, vgrid, dim3(256), 0, s, qv, mk, keys, nblk, pa, st_in, dg, res, pd, pb);
    // pb (sum of res) is consumed by k_cg_c before k_cg_c's own partials go to a third buffer
    hipLaunchKernelGGL(k_cg_c, vgrid, dim3(256), 0, s, mk, keys, nblk, pb, res, pb + (size_t)B * nblk);
    hipLaunchKernelGGL(k_cg_d, vgrid, dim3(256), 0, s, mk, keys, nblk, pb + (size_t)B * nblk, pa, tol2, st_in,
                       st_out, res, pd, pdf);
    st = hip_check("CG step launch");
    if (st != SK_OK) return st;
  }
  // 5. P [dg, dg q]
  hipLaunchKernelGGL(k_hvp_gmat, dim3(blocks_for(nk)), dim3(256), 0, s, Qraw, in16, dg, nk, d, keys, cen, mat);
  st = hip_check("HVP matrix launch");
  if (st == SK_OK) st = apply_plan(p, X, Y, w, L, pot_r, pot_k, lse_r, eps, side, mat, d + 1, gm, s);
  if (st != SK_OK) return st;
  // 6. sum_j P_ij (q_j . v_i) q_j = M_i v_i in one row-weighted plan pass
  st = apply_uw(p, X, Y, w, L, pot_r, pot_k, lse_r, eps, side, V, quad, s);
  if (st != SK_OK) return st;
  // 7. assemble
  hipLaunchKernelGGL(k_hvp_final, dim3(blocks_for(nr)), dim3(256), 0, s, Praw, in16, V, py, mr, zr, cr, gm, quad, nr,
                     d, rows, cen, (double)eps, out);
  return hip_check("HVP assembly launch");
}

sk_status init_impl(const sk_problem* p, const void* X, const void* Y, const float* a, const float* b, void* ws,
                    const Layout& L, hipStream_t stream) {
  char* w = static_cast<char*>(ws);
  const int B = (int)p->batch, d = (int)p->d;
  float* maxabs = reinterpret_cast<float*>(w + L.maxabs);
  double* cen = reinterpret_cast<double*>(w + L.cen);
  unsigned* box = reinterpret_cast<unsigned*>(w + L.box);
  unsigned* inexact = reinterpret_cast<unsigned*>(w + L.inexact);
  auto zero = [&](size_t off, size_t bytes) {
    const size_t n16 = bytes / 16;
    if (n16) hipLaunchKernelGGL(k_zero, dim3((unsigned)std::min<size_t>((n16 + 255) / 256, 4096)), dim3(256), 0,
                                stream, reinterpret_cast<u4*>(w + off), n16);
  };
  // box slots, bf16 centring flags, the status word and the key operands' lambda
  // tags (new clouds: the key operands hold no coordinate parts yet)
  hipLaunchKernelGGL(k_init_words, dim3((unsigned)std::min<long long>((4LL * B * d + 255) / 256, 1024)), dim3(256), 0,
                     stream, box, d, B, inexact, reinterpret_cast<unsigned*>(w + L.status),
                     reinterpret_cast<unsigned*>(w + L.ktag));
  if (L.cosine) {
    // normalised points: not centred, every coordinate at most 1 in magnitude
    zero(L.cen, align_up(8 * (size_t)B * d, 16));
    hipLaunchKernelGGL(k_fill_f32, dim3((2 * B + 255) / 256), dim3(256), 0, stream, maxabs, 2 * B, 1.f);
  } else {
    const int most = (int)std::max(p->n, p->m);
    // about 16 points per thread
    const int per = d <= 256 ? 256 / d : 1;
    // (at most 256 blocks per side and problem: each adds d minima and maxima to the same words)
    const unsigned chunks = (unsigned)std::min(256, std::max(1, (most + 16 * per - 1) / (16 * per)));
    hipLaunchKernelGGL(k_bbox, dim3(chunks, 2, B), dim3(256), 0, stream, X, Y, L.in_bf16, (int)p->n, (int)p->m, d,
                       box);
    hipLaunchKernelGGL(k_centre, dim3(B), dim3(256), 0, stream, box, d, B, L.in_bf16, 1, cen, maxabs, inexact);
    if (L.in_bf16) {
      const long long elems = (long long)most * d;  // about 8 elements per thread
      const unsigned ch = (unsigned)std::min<long long>(65535, std::max<long long>(1, (elems + 2047) / 2048));
      hipLaunchKernelGGL(k_bf16_exact, dim3(ch, B, 2), dim3(256), 0, stream, static_cast<const u16*>(X),
                         static_cast<const u16*>(Y), (long long)(p->n * p->d), (long long)(p->m * p->d), d, cen, inexact);
      hipLaunchKernelGGL(k_cen_fix, dim3(B), dim3(256), 0, stream, inexact, d, cen);
    }
  }
  auto side = [&](const void* P, const float* wt, int rows, int rows_pad, const float* mabs, size_t norm,
                  size_t logw, size_t rnorm, size_t op) {
    double* nrm = reinterpret_cast<double*>(w + norm);
    double* lw = reinterpret_cast<double*>(w + logw);
    double* rn = reinterpret_cast<double*>(w + rnorm);
    u16* dst = reinterpret_cast<u16*>(w + op);
    const dim3 rgrid((rows + 255) / 256, B);
    const dim3 ogrid((unsigned)(((long long)rows_pad * (L.KP / 8) + 255) / 256), B);
    if (L.mode == MODE_SPLIT) {
      hipLaunchKernelGGL(k_init_rows<MODE_SPLIT>, rgrid, dim3(256), 0, stream, P, wt, rows, d, L.in_bf16, L.cosine,
                         cen, nrm, lw, rn);
      hipLaunchKernelGGL(k_init_ops<MODE_SPLIT>, ogrid, dim3(256), 0, stream, P, rows, rows_pad, d, L.KP, L.in_bf16,
                         mabs, cen, rn, dst);
    } else if (L.mode == MODE_HILO) {
      hipLaunchKernelGGL(k_init_rows<MODE_HILO>, rgrid, dim3(256), 0, stream, P, wt, rows, d, L.in_bf16, L.cosine,
                         cen, nrm, lw, rn);
      hipLaunchKernelGGL(k_init_ops<MODE_HILO>, ogrid, dim3(256), 0, stream, P, rows, rows_pad, d, L.KP, L.in_bf16,
                         mabs, cen, rn, dst);
    } else {
      hipLaunchKernelGGL(k_init_rows<MODE_BF16>, rgrid, dim3(256), 0, stream, P, wt, rows, d, L.in_bf16, L.cosine,
                         cen, nrm, lw, rn);
      hipLaunchKernelGGL(k_init_ops<MODE_BF16>, ogrid, dim3(256), 0, stream, P, rows, rows_pad, d, L.KP, L.in_bf16,
                         mabs, cen, rn, dst);
    }
  };
  side(X, a, (int)p->n, L.n_pad, maxabs, L.xn, L.la, L.rx, L.qx);
  side(Y, b, (int)p->m, L.m_pad, maxabs + B, L.yn, L.lb, L.ry, L.qy);
  if (L.mode != MODE_SPLIT) {
    // bias vectors: padding keys (never written by a potential's epilogue)
    // remove themselves with the most negative bias
    const int nh0 = B * L.m_pad + SLACK, nh1 = B * L.n_pad + SLACK;
    hipLaunchKernelGGL(k_fill_f32, dim3((nh0 + 255) / 256), dim3(256), 0, stream,
                       reinterpret_cast<float*>(w + L.hb), nh0, NEG_BIG);
    hipLaunchKernelGGL(k_fill_f32, dim3((nh1 + 255) / 256), dim3(256), 0, stream,
                       reinterpret_cast<float*>(w + L.hb1), nh1, NEG_BIG);
  }
  // the slack rows after the last problem's operand rows: a workgroup whose
  // query rows run past the padding reads zeros there
  zero(L.qx + 2 * (size_t)B * L.n_pad * L.KP, 2 * (size_t)SLACK * L.KP);
  zero(L.qy + 2 * (size_t)B * L.m_pad * L.KP, 2 * (size_t)SLACK * L.KP);
  return hip_check("init kernel launch");
}

// Argument checks of the solve entry points (after the problem and workspace checks).
sk_status check_solve_args(const void* X, const void* Y, const float* a, const float* b, const float* eps,
                           int64_t n_eps, int64_t iters, const float* f, const float* g) {
  if (!X || !Y || !a || !b || !f || !g) {
    set_err("X, Y, a, b, f and g must be non-NULL device pointers");
    return SK_EINVAL;
  }
  if (iters < 0) {
    set_err("iters must be >= 0 (got %lld)", (long long)iters);
    return SK_EINVAL;
  }
  if (eps == nullptr || !(n_eps == 1 || (n_eps == iters && iters > 0))) {
    set_err("eps must be a host array of 1 or iters values (n_eps = %lld, iters = %lld)", (long long)n_eps,
            (long long)iters);
    return SK_EINVAL;
  }
  for (int64_t k = 0; k < n_eps; ++k)
    if (!eps_ok(eps[k])) {
      set_err("eps[%lld] must be positive and finite (got %g)", (long long)k, (double)eps[k]);
      return SK_EINVAL;
    }
  return SK_OK;
}

// init, then iters x (f half-step, g half-step), all enqueued on one stream.
// Each half-step writes the key bias its successor needs where it finalises
// its potential, so the successor launches no preparation kernel.  bf16 path:
// always (the bias is all that changes with the potential and eps).  fp32
// path: while eps stays the same, once the successor's key operand holds its
// coordinate parts for that eps (built by a preparation earlier in this solve);
// an eps change rebuilds them with a preparation kernel.
sk_status solve_impl(const sk_problem* p, const void* X, const void* Y, const float* a, const float* b,
                     const float* eps, int64_t n_eps, int64_t iters, float* f, float* g, void* ws, const Layout& L,
                     hipStream_t s) {
  sk_status st = init_impl(p, X, Y, a, b, ws, L, s);
  char* w = static_cast<char*>(ws);
  bool built[2] = {false, false};  // key operand of each side prepared in this solve ...
  float built_eps[2] = {0.f, 0.f};  // ... for this eps
  bool ready[2] = {false, false};   // its bias for the coming half-step already written
  auto writable = [&](int side, float e) {
    // bf16: the bias is all that changes; split and hi/lo: the key operand's
    // coordinate parts must already be built for this eps
    return L.mode == MODE_BF16 || (built[side] && built_eps[side] == e);
  };
  auto step = [&](int side, float e, bool has_next, float e_next) {
    const bool fuse = has_next && writable(1 - side, e_next);
    const NextBias nb = next_bias(p, w, L, side, e_next, fuse);
    const sk_status r = half_step(p, X, Y, ws, L, side == 0 ? g : f, e, side == 0 ? f : g, side, s, ready[side], nb);
    if (!ready[side]) {
      built[side] = true;
      built_eps[side] = e;
    }
    ready[side] = false;
    ready[1 - side] = fuse;
    return r;
  };
  for (int64_t k = 0; k < iters && st == SK_OK; ++k) {
    const float e = eps[n_eps == 1 ? 0 : k];
    const bool more = k + 1 < iters;
    const float e1 = more ? eps[n_eps == 1 ? 0 : k + 1] : e;
    st = step(0, e, true, e);
    if (st == SK_OK) st = step(1, e, more, e1);
  }
  return st;
}

// Device address of this device's copy of the built-in scratch array (see
// sinkhorn_solve_noalloc), looked up once per device with that device current.
sk_status scratch_address(void** out) {
  constexpr int MAX_DEV = 64;
  static std::mutex mu;
  static void* addr[MAX_DEV] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEV) {
    set_err("no usable current device (hipGetDevice failed or device index >= %d)", MAX_DEV);
    return SK_EHIP;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      set_err("hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
      return SK_EHIP;
    }
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return SK_OK;
}

}  // namespace

extern "C" {

size_t sinkhorn_workspace_bytes(const sk_problem* p) {
  if (check_problem(p) != SK_OK) return 0;
  return layout_of(p).total;
}

const char* sinkhorn_last_error(void) { return g_err; }

sk_status sinkhorn_init_norms(const sk_problem* p, const void* X, const void* Y, const float* a, const float* b,
                              void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  Layout L;
  sk_status st = check_ws(p, ws, ws_bytes, &L);
  if (st != SK_OK) return st;
  if (!X || !Y || !a || !b) {
    set_err("X, Y, a and b must be non-NULL device pointers");
    return SK_EINVAL;
  }
  return init_impl(p, X, Y, a, b, ws, L, static_cast<hipStream_t>(stream));
}

sk_status sinkhorn_half_step_f(const sk_problem* p, const void* X, const void* Y, void* ws, size_t ws_bytes,
                               const float* g, float eps, float* f, void* stream) {
  g_err[0] = 0;
  Layout L;
  sk_status st = check_ws(p, ws, ws_bytes, &L);
  if (st != SK_OK) return st;
  if (!X || !Y || !g || !f) {
    set_err("X, Y, g and f must be non-NULL device pointers");
    return SK_EINVAL;
  }
  if (!eps_ok(eps)) {
    set_err("eps must be positive and finite (got %g)", (double)eps);
    return SK_EINVAL;
  }
  return half_step(p, X, Y, ws, L, g, eps, f, 0, static_cast<hipStream_t>(stream));
}

sk_status sinkhorn_half_step_g(const sk_problem* p, const void* X, const void* Y, void* ws, size_t ws_bytes,
                               const float* f, float eps, float* g, void* stream) {
  g_err[0] = 0;
  Layout L;
  sk_status st = check_ws(p, ws, ws_bytes, &L);
  if (st != SK_OK) return st;
  if (!X || !Y || !g || !f) {
    set_err("X, Y, f and g must be non-NULL device pointers");
    return SK_EINVAL;
  }
  if (!eps_ok(eps)) {
    set_err("eps must be positive and finite (got %g)", (double)eps);
    return SK_EINVAL;
  }
  return half_step(p, X, Y, ws, L, f, eps, g, 1, static_cast<hipStream_t>(stream));
}

sk_status sinkhorn_solve(const sk_problem* p, const void* X, const void* Y, const float* a, const float* b,
                         const float* eps, int64_t n_eps, int64_t iters, float* f, float* g, void* ws,
                         size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  Layout L;
  sk_status st = check_ws(p, ws, ws_bytes, &L);
  if (st != SK_OK) return st;
  st = check_solve_args(X, Y, a, b, eps, n_eps, iters, f, g);
  if (st != SK_OK) return st;
  return solve_impl(p, X, Y, a, b, eps, n_eps, iters, f, g, ws, L, static_cast<hipStream_t>(stream));
}

sk_status sinkhorn_solve_noalloc(const sk_problem* p, const void* X, const void* Y, const float* a, const float* b,
                                 const float* eps, int64_t n_eps, int64_t iters, float* f, float* g,
                                 uint32_t* flags, void* stream) {
  g_err[0] = 0;
  sk_status st = check_problem(p);
  if (st != SK_OK) return st;
  const Layout L = layout_of(p);
  if (L.total > (size_t)SK_NOALLOC_MAX_BYTES) {
    set_err("problem needs %zu bytes of workspace, more than the %zu of the built-in scratch array "
            "(use sinkhorn_solve with a workspace)", L.total, (size_t)SK_NOALLOC_MAX_BYTES);
    return SK_EWORKSPACE;
  }
  st = check_solve_args(X, Y, a, b, eps, n_eps, iters, f, g);
  if (st != SK_OK) return st;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != SK_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = solve_impl(p, X, Y, a, b, eps, n_eps, iters, f, g, ws, L, s);
  if (st != SK_OK || flags == nullptr) return st;
  hipLaunchKernelGGL(k_copy_u32, dim3(1), dim3(64), 0, s,
                     reinterpret_cast<const unsigned*>(static_cast<char*>(ws) + L.status), flags);
  return hip_check("status copy launch");
}

sk_status sinkhorn_range_flags(const sk_problem* p, const void* ws, size_t ws_bytes, uint32_t* flags, void* stream) {
  g_err[0] = 0;
  Layout L;
  sk_status st = check_ws(p, const_cast<void*>(ws), ws_bytes, &L);
  if (st != SK_OK) return st;
  if (flags == nullptr) {
    set_err("flags must be a non-NULL device pointer");
    return SK_EINVAL;
  }
  hipLaunchKernelGGL(k_copy_u32, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                     reinterpret_cast<const unsigned*>(static_cast<const char*>(ws) + L.status), flags);
  return hip_check("status copy launch");
}

sk_status sinkhorn_marginal_error(const sk_problem* p, const void* X, const void* Y, void* ws, size_t ws_bytes,
                                  const float* f, const float* g, float eps, float* err, void* stream) {
  g_err[0] = 0;
  Layout L;
  sk_status st = check_ws(p, ws, ws_bytes, &L);
  if (st != SK_OK) return st;
  if (!X || !Y || !f || !g || !err) {
    set_err("X, Y, f, g and err must be non-NULL device pointers");
    return SK_EINVAL;
  }
  if (!eps_ok(eps)) {
    set_err("eps must be positive and finite (got %g)", (double)eps);
    return SK_EINVAL;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  float* tilde = reinterpret_cast<float*>(w + L.scratch);
  const int B = (int)p->batch;
  // rows: sum_j P_ij = a_i exp((f_i - T_f(g)_i)/eps)
  st = half_step(p, X, Y, ws, L, g, eps, tilde, 0, s);
  if (st != SK_OK) return st;
  hipLaunchKernelGGL(k_marginal, dim3(B), dim3(256), 0, s, f, tilde, reinterpret_cast<const double*>(w + L.la),
                     (int)p->n, 1.f / eps, err, 0);
  st = hip_check("marginal reduction launch");
  if (st != SK_OK) return st;
  // columns: sum_i P_ij = b_j exp((g_j - T_g(f)_j)/eps)
  st = half_step(p, X, Y, ws, L, f, eps, tilde, 1, s);
  if (st != SK_OK) return st;
  hipLaunchKernelGGL(k_marginal, dim3(B), dim3(256), 0, s, g, tilde, reinterpret_cast<const double*>(w + L.lb),
                     (int)p->m, 1.f / eps, err, 1);
  return hip_check("marginal reduction launch");
}

size_t sinkhorn_transport_workspace_bytes(const sk_problem* p) {
  if (check_problem(p) != SK_OK) return 0;
  return layout_of(p).ttotal;
}

static sk_status transport_entry(const sk_problem* p, const void* X, const void* Y, void* ws, size_t ws_bytes,
                                 const float* f, const float* g, float eps, float* bary, float* grad, void* stream,
                                 int side) {
  g_err[0] = 0;
  Layout L;
  sk_status st = check_ws(p, ws, ws_bytes, &L, 1);
  if (st != SK_OK) return st;
  if (!X || !Y || !f || !g || !bary) {
    set_err("X, Y, f, g and bary must be non-NULL device pointers");
    return SK_EINVAL;
  }
  if (!eps_ok(eps)) {
    set_err("eps must be positive and finite (got %g)", (double)eps);
    return SK_EINVAL;
  }
  return transport(p, X, Y, ws, L, f, g, eps, bary, grad, side, static_cast<hipStream_t>(stream));
}

sk_status sinkhorn_barycentric_x(const sk_problem* p, const void* X, const void* Y, void* ws, size_t ws_bytes,
                                 const float* f, const float* g, float eps, float* bary, float* grad, void* stream) {
  return transport_entry(p, X, Y, ws, ws_bytes, f, g, eps, bary, grad, stream, 0);
}

sk_status sinkhorn_barycentric_y(const sk_problem* p, const void* X, const void* Y, void* ws, size_t ws_bytes,
                                 const float* f, const float* g, float eps, float* bary, float* grad, void* stream) {
  return transport_entry(p, X, Y, ws, ws_bytes, f, g, eps, bary, grad, stream, 1);
}

static sk_status apply_entry(const sk_problem* p, const void* X, const void* Y, void* ws, size_t ws_bytes,
                             const float* f, const float* g, float eps, const float* M, int64_t c, float* out,
                             void* stream, int side) {
  g_err[0] = 0;
  Layout L;
  sk_status st = check_ws(p, ws, ws_bytes, &L, 1);
  if (st != SK_OK) return st;
  if (!X || !Y || !f || !g || !M || !out) {
    set_err("X, Y, f, g, the matrix and out must be non-NULL device pointers");
    return SK_EINVAL;
  }
  if (c < 1 || c > (int64_t)1 << 20) {
    set_err("columns c = %lld must be in 1 .. 2^20", (long long)c);
    return SK_EINVAL;
  }
  if (!eps_ok(eps)) {
    set_err("eps must be positive and finite (got %g)", (double)eps);
    return SK_EINVAL;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  float* lse = reinterpret_cast<float*>(w + L.scratch);
  st = half_step(p, X, Y, ws, L, side == 0 ? g : f, eps, lse, side, s);
  if (st != SK_OK) return st;
  return apply_plan(p, X, Y, w, L, side == 0 ? f : g, side == 0 ? g : f, lse, eps, side, M, (int)c, out, s);
}

sk_status sinkhorn_apply_plan_x(const sk_problem* p, const void* X, const void* Y, void* ws, size_t ws_bytes,
                                const float* f, const float* g, float eps, const float* V, int64_t c, float* out,
                                void* stream) {
  return apply_entry(p, X, Y, ws, ws_bytes, f, g, eps, V, c, out, stream, 0);
}

sk_status sinkhorn_apply_plan_y(const sk_problem* p, const void* X, const void* Y, void* ws, size_t ws_bytes,
                                const float* f, const float* g, float eps, const float* U, int64_t c, float* out,
                                void* stream) {
  return apply_entry(p, X, Y, ws, ws_bytes, f, g, eps, U, c, out, stream, 1);
}

size_t sinkhorn_hvp_workspace_bytes(const sk_problem* p) {
  if (check_problem(p) != SK_OK) return 0;
  return layout_of(p).htotal;
}

static sk_status hvp_entry(const sk_problem* p, const void* X, const void* Y, void* ws, size_t ws_bytes,
                           const float* f, const float* g, float eps, const float* V, int64_t cg_iters, float cg_tol,
                           float* out, void* stream, int side) {
  g_err[0] = 0;
  Layout L;
  sk_status st = check_ws(p, ws, ws_bytes, &L, 2);
  if (st != SK_OK) return st;
  if (!X || !Y || !f || !g || !V || !out) {
    set_err("X, Y, f, g, V and out must be non-NULL device pointers");
    return SK_EINVAL;
  }
  if (!eps_ok(eps)) {
    set_err("eps must be positive and finite (got %g)", (double)eps);
    return SK_EINVAL;
  }
  if (cg_iters < 0 || cg_iters > 100000 || !(cg_tol >= 0.f) || !isfinite(cg_tol)) {
    set_err("cg_iters must be in 0 .. 100000 and cg_tol >= 0 finite (got %lld, %g)", (long long)cg_iters,
            (double)cg_tol);
    return SK_EINVAL;
  }
  if (L.cosine) {
    set_err("Hessian-vector products support the squared-Euclidean cost only");
    return SK_EUNSUPPORTED;
  }
  return hvp(p, X, Y, static_cast<char*>(ws), L, f, g, eps, V, cg_iters, cg_tol, out, side,
             static_cast<hipStream_t>(stream));
}

sk_status sinkhorn_hvp_x(const sk_problem* p, const void* X, const void* Y, void* ws, size_t ws_bytes,
                         const float* f, const float* g, float eps, const float* V, int64_t cg_iters, float cg_tol,
                         float* out, void* stream) {
  return hvp_entry(p, X, Y, ws, ws_bytes, f, g, eps, V, cg_iters, cg_tol, out, stream, 0);
}

sk_status sinkhorn_hvp_y(const sk_problem* p, const void* X, const void* Y, void* ws, size_t ws_bytes,
                         const float* f, const float* g, float eps, const float* V, int64_t cg_iters, float cg_tol,
                         float* out, void* stream) {
  return hvp_entry(p, X, Y, ws, ws_bytes, f, g, eps, V, cg_iters, cg_tol, out, stream, 1);
}

}  // extern "C"
