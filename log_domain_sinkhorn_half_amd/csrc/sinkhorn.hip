// Log-domain Sinkhorn half-steps for squared-Euclidean cost on MI355X (gfx950).
//
// Method: page "FlashSinkhorn: IO-aware entropic OT on GPU", section
// "Methodology".  Part 1 (Proposition 1) rewrites the stabilised update
//   f_i <- -eps LSE_j[(g_j - C_ij)/eps + log b_j],  C_ij = ||x_i - y_j||^2
// as f_i = ||x_i||^2 - eps * LSE_j[(2 x_i.y_j + beta_j)/eps] with the per-column
// bias beta_j = g_j - ||y_j||^2 + eps log b_j: a dot-product score matrix with a
// bias, reduced by a row log-sum-exp.  Part 2 streams it: query tiles stay on
// chip (row-stationary), key tiles stream past them, the LSE is accumulated
// online and the n x m scores never reach HBM.  The g update is the same
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
// Beyond the half-step (same page, section "Differentiation and second-order
// optimisation"; and the closing remarks on costs):
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

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

namespace {

constexpr int MODE_SPLIT = 0;  // fp32 inputs
constexpr int MODE_BF16 = 1;   // bf16 inputs
constexpr int ROW_PAD = 512;   // operand buffers are padded to a multiple of this many rows
constexpr int KS_MAX = 64;     // most key splits per half-step
constexpr int SLACK = 256;     // slack rows after operand buffers (>= one chunk)
constexpr float NEG_BIG = -1e30f;
constexpr double LOG2E = 1.4426950408889634;
// Largest partial sum a lane may carry past a chunk check.  Kept well below
// FLT_MAX so that merging 4 lanes and up to KS_MAX key splits cannot overflow.
constexpr float SUM_LIMIT = 0x1p112f;
// Offsets sit this far (base 2) above the largest score seen when they are set:
// terms more than HEADROOM + 126 below it flush to zero (relative size below
// 2^-62 of that score's term), and scores may grow by HEADROOM + 112 before a
// chunk must be redone.
constexpr float HEADROOM = 64.f;
// Below this many keys the d <= 3 half-step uses SMALL_TC key tiles per chunk.
constexpr int SMALL_KEYS = 16384;
constexpr int SMALL_TC = 4;
// Key-operand segments per thread of k_prep_keys when every segment is rebuilt
// (1: the most parallel; measured fastest for full rebuilds).
constexpr int PREP_SEGS = 1;
constexpr int NXCD = 8;  // accelerator complex dies, each with its own L2
constexpr int gcd_c(int a, int b) { return b == 0 ? a : gcd_c(b, a % b); }

// ---------------------------------------------------------------------------
// K-slot layout of the fp32 path for point dimension d.
//   slots 0,1      query: -m (two bf16 parts, set in registers)    key: 1, 1
//   slots 2,3,4    query: 1, 1, 1                                   key: grid bias in 3 parts
//   slots 5..5+d-1 query: x_g[t]                                    key: v_g[t]
//   (pad to the correction start)
//   cb+7t+0..6     query: x_g x_g x_1 x_2 x_1 x_1 x_2               key: v_1 v_2 v_g v_g v_1 v_2 v_1
//   cb+7d, +1      query: 1, 1                                      key: bias remainder in 2 parts
// The grid section is exact in fp32; for d <= 3 it fills lane group 0 and the
// corrections fill groups 1-3 of a single MFMA; otherwise each section starts
// on an MFMA (32-slot) boundary so the grid sum is complete before any
// correction is added.
// ---------------------------------------------------------------------------
__host__ __device__ constexpr int split_grid_slots(int d) { return d + 5; }
__host__ __device__ constexpr int split_corr_slots(int d) { return 7 * d + 2; }
__host__ __device__ constexpr bool split_single(int d) { return split_grid_slots(d) <= 8 && split_corr_slots(d) <= 24; }
__host__ __device__ constexpr int split_corr_begin(int d) {
  return split_single(d) ? 8 : (split_grid_slots(d) + 31) / 32 * 32;
}
__host__ __device__ constexpr int split_nch(int d) {
  return split_single(d) ? 1 : (split_corr_begin(d) + split_corr_slots(d) + 31) / 32;
}
constexpr int MAX_NCH_SPLIT = split_nch(SK_MAX_D_FP32);
constexpr int MAX_NCH_BF16 = (SK_MAX_D + 31) / 32;

thread_local char g_err[512] = "";

void set_err(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
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
// Largest |coordinate| of each problem's X (side 0) and Y (side 1): a strided
// block reduction, then atomicMax on the float bits (values are >= 0, so the
// unsigned order is the float order).  maxabs must be zero beforehand.
__global__ __launch_bounds__(256) void k_maxabs(const void* __restrict__ X, const void* __restrict__ Y, int in_bf16,
                                                long long nx, long long ny, unsigned* __restrict__ maxabs,
                                                int batch) {
  __shared__ float red[256];
  const int b = blockIdx.y, side = blockIdx.z;
  const long long cnt = side == 0 ? nx : ny;
  const void* P = side == 0 ? X : Y;
  float mx = 0.f;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < cnt; i += (long long)gridDim.x * 256) {
    const long long k = (long long)b * cnt + i;
    mx = fmaxf(mx, fabsf(coord(P, (size_t)k, in_bf16)));
  }
  red[threadIdx.x] = mx;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  if (threadIdx.x == 0) atomicMax(&maxabs[side * batch + b], __float_as_uint(red[0]));
}

// Norms (fp64), log-weights (fp64), inverse norms and operand rows of one
// cloud: the split query layout (fp32 inputs, or any input under the cosine
// cost, whose points are first divided by their norm) or a zero-padded bf16
// copy (bf16 inputs, squared-Euclidean cost).
template <int MODE>
__global__ __launch_bounds__(256) void k_init_side(const void* __restrict__ P, const float* __restrict__ w,
                                                   int rows, int rows_pad, int d, int KP, int in_bf16, int cosine,
                                                   const float* __restrict__ maxabs, double* __restrict__ norm,
                                                   double* __restrict__ logw, double* __restrict__ rnorm,
                                                   u16* __restrict__ opnd) {
  const int b = blockIdx.y;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows_pad) return;
  u16* dst = opnd + ((size_t)b * rows_pad + i) * KP;
  if (i >= rows) {
    for (int k = 0; k < KP; k += 8) *reinterpret_cast<u4*>(dst + k) = u4{0, 0, 0, 0};
    return;
  }
  const size_t r = (size_t)b * rows + i;
  if (MODE == MODE_BF16) {
    const u16* src = static_cast<const u16*>(P) + r * d;
    double nrm = 0.0;
    for (int t = 0; t < d; ++t) {
      const double v = bf16_f(src[t]);
      nrm += v * v;
    }
    norm[r] = nrm;
    rnorm[r] = 1.0;
    logw[r] = log((double)w[r]);
    for (int k = 0; k < KP; k += 2) {
      const uint32_t lo = (k < d) ? src[k] : 0, hi = (k + 1 < d) ? src[k + 1] : 0;
      *reinterpret_cast<uint32_t*>(dst + k) = lo | (hi << 16);
    }
    return;
  }
  const int qe = grid_exponent(maxabs[b]);
  const double q = ldexp(1.0, qe), iq = ldexp(1.0, -qe);
  double rn = 1.0;
  if (cosine) {
    double raw = 0.0;
    for (int t = 0; t < d; ++t) {
      const double v = coord(P, r * d + t, in_bf16);
      raw += v * v;
    }
    rn = raw > 0.0 ? 1.0 / sqrt(raw) : 0.0;  // a zero point stays zero
  }
  auto val = [&](int t) { return (double)coord(P, r * d + t, in_bf16) * rn; };
  double nrm = 0.0;
  for (int t = 0; t < d; ++t) nrm += val(t) * val(t);
  norm[r] = nrm;
  rnorm[r] = rn;
  logw[r] = log((double)w[r]);
  const int cb = split_corr_begin(d);
  for (int k0 = 0; k0 < KP; k0 += 8) {
    u16 v[8];
    for (int e = 0; e < 8; ++e) {
      const int k = k0 + e;
      u16 v_ = 0;
      if (k >= 2 && k <= 4) {
        v_ = BF16_ONE;
      } else if (k >= 5 && k < 5 + d) {
        v_ = grid_split(val(k - 5), q, iq).g;
      } else if (k >= cb && k < cb + 7 * d) {
        const Parts pp = grid_split(val((k - cb) / 7), q, iq);
        const int s = (k - cb) % 7;
        v_ = (s <= 1) ? pp.g : ((s == 3 || s == 6) ? pp.r2 : pp.r1);
      } else if (k == cb + 7 * d || k == cb + 7 * d + 1) {
        v_ = BF16_ONE;
      }
      v[e] = v_;
    }
    *reinterpret_cast<u4*>(dst + k0) = u4{(uint32_t)v[0] | ((uint32_t)v[1] << 16), (uint32_t)v[2] | ((uint32_t)v[3] << 16),
                                         (uint32_t)v[4] | ((uint32_t)v[5] << 16), (uint32_t)v[6] | ((uint32_t)v[7] << 16)};
  }
}

// Grid and remainder parts of v = l2*y*rn (l2 = 2*lambda) for the key operand,
// in fp32: v is carried as vh + vl, exactly when rn == 1 (the product of two
// fp32 numbers and its fma error term), so the remainder takes one fp32
// rounding, as in the fp64 split.  q = 2^k and iq = 1/q must be normal floats.
__device__ __forceinline__ Parts key_split(float y, double rn, float l2, float q, float iq) {
  float vh, vl;
  if (rn == 1.0) {
    vh = l2 * y;
    vl = fmaf(l2, y, -vh);
  } else {
    const double v = (double)l2 * (double)y * rn;
    vh = (float)v;
    vl = (float)(v - (double)vh);
  }
  const float g = rintf(vh * iq) * q;
  const float r = (vh - g) + vl;  // vh - g is exact: both are multiples of ulp(vh)
  Parts p;
  p.g = bf16_rne(g);
  p.r1 = bf16_rne(r);
  p.r2 = bf16_rne(r - bf16_f(p.r1));
  return p;
}

// Bias lambda*(pot - norm + eps*logw) of key r in parts: bp[0..2] its multiple
// of the grid quantum Q (exact in three bf16 parts), bp[3..4] the remainder.
// Keys of zero weight and padding keys (real == false) take NEG_BIG alone.
__device__ __forceinline__ void bias_parts(bool real, size_t r, const float* __restrict__ pot,
                                           const double* __restrict__ norm, const double* __restrict__ logw,
                                           float lam, float eps, double Q, double iQ, u16 (&bp)[5]) {
  double bias = (double)NEG_BIG;
  if (real) {
    bias = (double)lam * ((double)pot[r] - norm[r] + (double)eps * logw[r]);
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
                                                   const double* __restrict__ rnorm, const float* __restrict__ pot,
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
      bias_parts(j < keys, (size_t)b * keys + j, pot, norm, logw, lam, eps, Q, iQ, bp);
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
      const float y = coord(P, r * d + t, in_bf16);
      return f32 ? key_split(y, rn, l2f, qkf, iqkf) : grid_split(lam2 * (double)y * rn, qk, iqk);
    };
    u16 bp[5] = {0, 0, 0, 0, 0};
    if (seg == 0 || seg == sb1 || seg == sb2) bias_parts(real, r, pot, norm, logw, lam, eps, Q, iQ, bp);
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

// Half bias (pot - norm + eps*logw)/2 per key (bf16 inputs); padding -> -1e30.
__global__ __launch_bounds__(256) void k_prep_bias(const float* __restrict__ pot, const double* __restrict__ norm,
                                                   const double* __restrict__ logw, int keys, int keys_pad,
                                                   float eps, float* __restrict__ hb) {
  const int b = blockIdx.y;
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= keys_pad) return;
  float v = NEG_BIG;
  if (j < keys) {
    const size_t r = (size_t)b * keys + j;
    v = (float)(0.5 * ((double)pot[r] - norm[r] + (double)eps * logw[r]));
    if (!(v >= NEG_BIG)) v = NEG_BIG;
  }
  hb[(size_t)b * keys_pad + j] = v;
}

// ---------------------------------------------------------------------------
// The streaming half-step kernel
// ---------------------------------------------------------------------------
typedef float f16v __attribute__((ext_vector_type(16)));

__device__ __forceinline__ bf16x8 as_bf16x8(u4 v) { return __builtin_bit_cast(bf16x8, v); }

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
// and, on the fp32 path, a multiple of the grid quantum Q.
__device__ __forceinline__ float offset_from_max(float mx, float Q) {
  float mq = floorf(mx);
  if (!(fabsf(mq) < 1e30f)) return mq;
  float quantum = fmaxf(Q, 1.f);
  if (fabsf(mq) >= 65536.f) quantum = fmaxf(quantum, ldexpf(1.f, ilogbf(mq) - 15));
  return floorf(mq / quantum) * quantum;
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

// TCX overrides the key tiles per chunk (0: cfg_TC), for small problems.
template <int MODE, int NCH, int TCX = 0>
__global__ __launch_bounds__(64 * cfg_NW(MODE, NCH)) __attribute__((amdgpu_waves_per_eu(cfg_waves(MODE, NCH)))) void k_lse(
    const u16* __restrict__ Q, const u16* __restrict__ K, const float* __restrict__ hb,
    const float* __restrict__ qgrid, const double* __restrict__ qnorm, float* __restrict__ out,
    float2* __restrict__ part, int rows, int rows_pad, int keys, int keys_pad, int chunks_per_split, int batch,
    float lam2, double inv_lam, unsigned* __restrict__ tag, unsigned tag_val) {
  constexpr int MW = cfg_MW(MODE, NCH), R = cfg_R(MODE, NCH), TC = TCX ? TCX : cfg_TC(MODE, NCH);
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
  // the last workgroup's query rows may run past the padded rows into the slack rows
  static_assert(NW * QPW - gcd_c(NW * QPW, ROW_PAD) <= SLACK, "query over-read beyond the slack rows");
  static_assert(CK % 4 == 0 && CK / 4 <= NT, "one 4-key bias vector per thread");
  // chunks must tile the padded key range: keys past it (slack rows) are not prepared
  static_assert(ROW_PAD % CK == 0 && CK <= SLACK, "a key chunk must divide the row padding");
  // One spare row per buffer takes the stores of threads past the end of a chunk.
  __shared__ __attribute__((aligned(16))) u16 lds[2][(CK + 1) * LROW];
  __shared__ __attribute__((aligned(16))) float ldsb[2][CK];

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
    m[c] = -FLT_MAX;
    s[c] = 0.f;
  }

  u4 pre[2][NLD];
  f4 preb[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  // Loads past the end of a chunk land in the slack rows that follow every
  // operand buffer, so they need no guard; their LDS stores go to a spare row.
  auto gload = [&](int chunk, auto par) {
    constexpr int P = decltype(par)::value;
    const u16* src = Kb + (size_t)chunk * CK * KP;
#pragma unroll
    for (int i = 0; i < NLD; ++i) pre[P][i] = *reinterpret_cast<const u4*>(src + (size_t)(tid + NT * i) * 8);
    if (MODE == MODE_BF16) preb[P] = *reinterpret_cast<const f4*>(hbb + (size_t)chunk * CK + (tid % (CK / 4)) * 4);
  };
  auto lstore = [&](auto par) {
    constexpr int P = decltype(par)::value;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int v = min(tid + NT * i, NVEC);  // NVEC maps to the spare row
      *reinterpret_cast<u4*>(&lds[P][(v / VPR) * LROW + (v % VPR) * 8]) = pre[P][i];
    }
    if (MODE == MODE_BF16 && tid < CK / 4) *reinterpret_cast<f4*>(&ldsb[P][tid * 4]) = preb[P];
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
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const u4 ka = *reinterpret_cast<const u4*>(&lds[buf][(t * MW + col) * LROW + i * T::KI + grp * 8]);
#pragma unroll
      for (int c = 0; c < R; ++c) acc[c] = T::mma(ka, bq[c][i], acc[c]);
    }
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
#pragma unroll
      for (int c = 0; c < R; ++c) {
        float mx = -INFINITY;
#pragma unroll
        for (int o = 0; o < NO; ++o) mx = fmaxf(mx, raw(acc[c][o]));
        m[c] = offset_from_max(lanes_max(mx) + HEADROOM, qg);
        if (MODE == MODE_SPLIT) set_offset(bq[c][0], -m[c], grp == 0);
      }
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
#pragma unroll
      for (int c = 0; c < R; ++c) {
        mx[c] = lanes_max(mx[c]);
        const float mn = fmaxf(m[c], offset_from_max(mx[c] + HEADROOM, qg));
        s[c] = rescale(s[c], m[c], mn);
        m[c] = mn;
        if (MODE == MODE_SPLIT) set_offset(bq[c][0], -m[c], grp == 0);
      }
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

#pragma unroll
  for (int c = 0; c < R; ++c) {
    const float st = lanes_sum(s[c]);
    const int q = qbase + MW * c + col;
    if (grp == 0 && q < rows) {
      const size_t r = (size_t)b * rows + q;
      if (part != nullptr) {
        part[(size_t)blk.y * batch * rows + r] = make_float2(m[c], st);
      } else {
        out[r] = (float)(qnorm[r] - ((double)m[c] + log2((double)st)) * inv_lam);
      }
    }
  }
}

// Merge the (max, sum) pairs of the key splits (one pass, exact power-of-two
// rescaling) and write the potential.
__global__ __launch_bounds__(256) void k_merge(const float2* __restrict__ part, int ks, int total,
                                               const double* __restrict__ qnorm, float* __restrict__ out,
                                               double inv_lam) {
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
  out[i] = (float)(qnorm[i] - ((double)M + log2((double)S)) * inv_lam);
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
// Transport application (page "FlashSinkhorn: IO-aware entropic OT on GPU",
// section "Differentiation and second-order optimisation"): the barycentric
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
constexpr int VK = 32;  // keys per value block: one 16x16x32 K step, two 16-key score tiles

__host__ __device__ constexpr int val_parts(int mode) { return mode == MODE_SPLIT ? 3 : 1; }
__host__ __device__ constexpr int val_tiles(int mode, int d) { return (val_parts(mode) * d + 15) / 16; }
// A spare value column holds ones, so the P.V product also yields the sum of the weights.
__host__ __device__ constexpr bool val_sumcol(int mode, int d) { return val_parts(mode) * d < val_tiles(mode, d) * 16; }
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
// 32-key value blocks per LDS chunk of the transport kernel (fewer barriers for small operands)
__host__ __device__ constexpr int bary_TCB(int nch, int nct) { return (nch <= 2 && nct <= 4) ? 4 : 1; }

__device__ __forceinline__ u4 pack8(const u16 (&v)[8]) {
  return u4{(uint32_t)v[0] | ((uint32_t)v[1] << 16), (uint32_t)v[2] | ((uint32_t)v[3] << 16),
            (uint32_t)v[4] | ((uint32_t)v[5] << 16), (uint32_t)v[6] | ((uint32_t)v[7] << 16)};
}

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
__global__ __launch_bounds__(256) void k_prep_vals(const void* __restrict__ P, int mode, int in_bf16,
                                                   const double* __restrict__ rnorm, int keys, int keys_pad, int d,
                                                   int ncols, int sumcol, u16* __restrict__ vt) {
  const int b = blockIdx.y;
  const long long per_blk = (long long)ncols * (VK / 8);
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)(keys_pad / VK) * per_blk) return;
  const int blk = (int)(idx / per_blk);
  const int rem = (int)(idx % per_blk);
  const int c = rem / (VK / 8), k0 = (rem % (VK / 8)) * 8;
  const int part = c / d, t = c % d;
  u16 v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int j = blk * VK + vkey(k0, e);
    u16 val = 0;
    if (j < keys && sumcol && c == ncols - 1) {
      val = BF16_ONE;
    } else if (j < keys && part < val_parts(mode)) {
      const size_t r = ((size_t)b * keys + j) * d + t;
      if (mode == MODE_BF16) {
        val = static_cast<const u16*>(P)[r];
      } else {
        // x = h0 + h1 + h2 exactly: each remainder is exact in fp32
        const float x = (float)((double)coord(P, r, in_bf16) * rnorm[(size_t)b * keys + j]);
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
    unsigned tag_val, const u16* __restrict__ U, float ugain) {
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
      const float mo = offset_from_max((float)M, qg);
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
        if (__any(first || wm > __float_as_uint(0x1p32f))) {
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
            if (mo[c] == -INFINITY || !(top - mo[c] <= 32.f)) mn = fmaxf(mo[c], offset_from_max(top + HEADROOM, qg));
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

// Barycentric projection and gradient from the split partials, one thread per
// (problem, row, coordinate): bary = sum_parts sum_splits pv / sum_splits s,
// grad = 2 r (p - bary) with the row mass r = w exp((pot - lse)/eps).
// With lazy offsets (mpart != nullptr) each split's partials are relative to its
// own offset mpart (base 2): they are brought to the largest one, and the row's
// log-sum-exp follows from it and the weight sum, as in the half-step:
// lse = ||p||^2 - (M + log2 S) / lambda, written to lse for later passes.
__global__ __launch_bounds__(256) void k_bary_merge(const float* __restrict__ pv, const float* __restrict__ sp, int ks,
                                                    int batch, int rows, int d, int ncols, int parts, int sumcol,
                                                    const void* __restrict__ P, int in_bf16,
                                                    const float* __restrict__ pot, float* __restrict__ lse,
                                                    const double* __restrict__ logw, double eps,
                                                    const float* __restrict__ mpart, const double* __restrict__ qnorm,
                                                    double inv_lam, float* __restrict__ bary,
                                                    float* __restrict__ grad) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)batch * rows * d) return;
  const int t = (int)(idx % d);
  const long long rr = idx / d;  // b * rows + row
  double M = 0.0;
  if (mpart != nullptr) {
    M = -INFINITY;
#pragma unroll 4
    for (int k = 0; k < ks; ++k) M = fmax(M, (double)mpart[(size_t)k * batch * rows + (size_t)rr]);
  }
  double S = 0.0, num = 0.0;
#pragma unroll 4
  for (int k = 0; k < ks; ++k) {
    const size_t base = (size_t)k * batch * rows + (size_t)rr;
    const double sc = mpart != nullptr ? exp2((double)mpart[base] - M) : 1.0;  // 0 for an empty split
    S += sc * (sumcol ? (double)pv[base * ncols + ncols - 1] : (double)sp[base]);
    for (int part = 0; part < parts; ++part) num += sc * (double)pv[base * ncols + part * d + t];
  }
  const double bc = num / S;
  bary[idx] = (float)bc;
  double row_lse;
  if (mpart != nullptr) {
    row_lse = qnorm[rr] - (M + log2(S)) * inv_lam;
    if (t == 0) lse[rr] = (float)row_lse;
  } else {
    row_lse = (double)lse[rr];
  }
  if (grad != nullptr) {
    const double x = coord(P, (size_t)idx, in_bf16);
    const double mass = exp(logw[rr] + ((double)pot[rr] - row_lse) / eps);
    grad[idx] = (float)(2.0 * mass * (x - bc));
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
// Plan application and Hessian-vector products (page "FlashSinkhorn: IO-aware
// entropic OT on GPU", section "Differentiation and second-order
// optimisation": the Hessian-vector product decomposes into vector- and
// matrix-transport products, so neither the Hessian nor the plan is formed).
// A plan application out_i = sum_j P_ij V_j is the transport pass above with V
// an arbitrary fp32 matrix, scaled by the row mass.
// ---------------------------------------------------------------------------
constexpr int APPLY_COLS = 64;  // matrix columns per pass (3 parts each + the ones column <= 13 tiles)

__host__ __device__ constexpr int apply_tiles(int cb) { return cb <= 5 ? 1 : (cb <= 21 ? 4 : 13); }

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
__global__ __launch_bounds__(256) void k_apply_merge(const float* __restrict__ pv, int ks, int batch, int rows, int cb,
                                                     int ncols, int c, int col0, const double* __restrict__ logw,
                                                     const float* __restrict__ pot, const float* __restrict__ lse,
                                                     double eps, float* __restrict__ out) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)batch * rows * cb) return;
  const int k = (int)(idx % cb);
  const long long rr = idx / cb;
  double S = 0.0, num = 0.0;
#pragma unroll 4
  for (int sp = 0; sp < ks; ++sp) {
    const size_t base = ((size_t)sp * batch * rows + (size_t)rr) * ncols;
    S += (double)pv[base + ncols - 1];
    for (int part = 0; part < 3; ++part) num += (double)pv[base + part * cb + k];
  }
  const double mass = exp(logw[rr] + ((double)pot[rr] - (double)lse[rr]) / eps);
  out[rr * c + col0 + k] = (float)(mass > 0.0 ? mass * num / S : 0.0);
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
                                                  long long total, int d, double* __restrict__ zr,
                                                  double* __restrict__ cr, float* __restrict__ M) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  double z = 0.0, vpy = 0.0;
  for (int t = 0; t < d; ++t) {
    const double v = V[i * d + t];
    z += (double)coord(P, (size_t)i * d + t, in_bf16) * v;
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
                                                 long long total, int d, double* __restrict__ rhs) {
  const long long j = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= total) return;
  const float* w = W + j * (d + 2);
  double qw = 0.0;
  for (int t = 0; t < d; ++t) qw += (double)coord(Q, (size_t)j * d + t, in_bf16) * (double)w[1 + t];
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
constexpr int CG_BLK = 2048;

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
                                                  const double* __restrict__ dg, long long total, int d,
                                                  float* __restrict__ M) {
  const long long j = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= total) return;
  float* row = M + j * (d + 1);
  row[0] = (float)dg[j];
  for (int t = 0; t < d; ++t) row[1 + t] = (float)(dg[j] * (double)coord(Q, (size_t)j * d + t, in_bf16));
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
                                                  int batch, int rows, int d, int ncols, int parts,
                                                  const double* __restrict__ logw, const float* __restrict__ pot,
                                                  const float* __restrict__ lse, double eps,
                                                  double* __restrict__ quad) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)batch * rows * d) return;
  const int t = (int)(idx % d);
  const long long rr = idx / d;
  double S = 0.0, num = 0.0;
#pragma unroll 4
  for (int k = 0; k < ks; ++k) {
    const size_t base = (size_t)k * batch * rows + (size_t)rr;
    S += (double)sp[base];
    for (int part = 0; part < parts; ++part) num += (double)pv[base * ncols + part * d + t];
  }
  const double mass = exp(logw[rr] + ((double)pot[rr] - (double)lse[rr]) / eps);
  quad[idx] = mass > 0.0 ? mass * num / S : 0.0;
}

// Coordinates of a cloud as an fp32 matrix.
__global__ __launch_bounds__(256) void k_coords(const void* __restrict__ P, int in_bf16, long long total,
                                                float* __restrict__ M) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < total) M[i] = coord(P, (size_t)i, in_bf16);
}

// HV_i = 2 r v + (2/eps) [ df (r p - PY) + p (P dg) - P(dg q) - 2 (z (r p - PY) - (v.PY) p + quad) ]
// with df = (cr - P dg)/r; G = P [dg, dg q].
__global__ __launch_bounds__(256) void k_hvp_final(const void* __restrict__ P, int in_bf16,
                                                   const float* __restrict__ V, const float* __restrict__ PY,
                                                   const double* __restrict__ mass, const double* __restrict__ zr,
                                                   const double* __restrict__ cr, const float* __restrict__ G,
                                                   const double* __restrict__ quad, long long total, int d,
                                                   double eps, float* __restrict__ out) {
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
    const double pt = coord(P, (size_t)i * d + t, in_bf16);
    const double grad_half = r * pt - (double)PY[i * d + t];
    const double K = 2.0 * (z * grad_half - vpy * pt + quad[i * d + t]);
    const double inner = df * grad_half + pt * (double)g[0] - (double)g[1 + t] - K;
    out[i * d + t] = (float)(2.0 * r * (double)V[i * d + t] + (2.0 / eps) * inner);
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
struct Layout {
  int mode, KP, n_pad, m_pad, max_pad;
  int in_bf16, cosine;
  size_t xn, yn, la, lb, rx, ry, maxabs, qgrid, ktag, qx, qy, kbx, kby, hb, part, scratch, total;
  // key operand of the fp32 path for side 0 (Y as keys) or side 1 (X as keys)
  size_t kb(int side) const { return side == 0 ? kby : kbx; }
  // transport application and plan products (after `total`; only their entry points need them)
  int ncols;             // widest value operand (columns) of any transport pass
  size_t bpv_bytes;      // bytes of the split-partials region
  size_t vt, bpv, bs, bm, ttotal;
  // Hessian-vector products (after `ttotal`)
  size_t h_lse_r, h_lse_k, h_mr, h_mk, h_py, h_mat, h_w, h_g, h_quad, h_zr, h_cr, h_rhs, h_dg, h_res,
      h_pd, h_pdf, h_t, h_q, h_st, h_part, h_u, htotal;
};

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int kp_for(int mode, int64_t d) {
  if (mode == MODE_SPLIT) return split_nch((int)d) * 32;
  return (int)align_up((size_t)d, 32);
}

sk_status check_problem(const sk_problem* p) {
  if (p == nullptr) {
    set_err("problem descriptor is NULL");
    return SK_EINVAL;
  }
  if (p->dtype != SK_FP32 && p->dtype != SK_BF16) {
    set_err("unknown dtype %d (expected SK_FP32=0 or SK_BF16=1)", (int)p->dtype);
    return SK_EDTYPE;
  }
  if (p->batch < 1 || p->n < 1 || p->m < 1 || p->d < 1) {
    set_err("batch, n, m and d must be >= 1 (got %lld, %lld, %lld, %lld)", (long long)p->batch,
            (long long)p->n, (long long)p->m, (long long)p->d);
    return SK_ESHAPE;
  }
  if (p->d > SK_MAX_D) {
    set_err("d = %lld exceeds SK_MAX_D = %d", (long long)p->d, SK_MAX_D);
    return SK_EUNSUPPORTED;
  }
  if (p->cost != SK_COST_SQEUCLID && p->cost != SK_COST_COSINE) {
    set_err("unknown cost %d (expected SK_COST_SQEUCLID=0 or SK_COST_COSINE=1)", (int)p->cost);
    return SK_EINVAL;
  }
  if ((p->dtype == SK_FP32 || p->cost == SK_COST_COSINE) && p->d > SK_MAX_D_FP32) {
    set_err("d = %lld exceeds SK_MAX_D_FP32 = %d for fp32 inputs and the cosine cost", (long long)p->d,
            SK_MAX_D_FP32);
    return SK_EUNSUPPORTED;
  }
  const int64_t lim = (int64_t)1 << 30;
  if (p->n >= lim || p->m >= lim || p->batch >= 65536 || p->batch * std::max(p->n, p->m) >= ((int64_t)1 << 31)) {
    set_err("problem too large (batch*max(n,m) must stay below 2^31, batch < 65536)");
    return SK_ESHAPE;
  }
  return SK_OK;
}

Layout layout_of(const sk_problem* p) {
  Layout L{};
  L.in_bf16 = p->dtype == SK_BF16;
  L.cosine = p->cost == SK_COST_COSINE;
  // bf16 operands are used as they are; fp32 inputs and normalised points take the split layout
  L.mode = (L.in_bf16 && !L.cosine) ? MODE_BF16 : MODE_SPLIT;
  L.KP = kp_for(L.mode, p->d);
  L.n_pad = (int)align_up((size_t)p->n, ROW_PAD);
  L.m_pad = (int)align_up((size_t)p->m, ROW_PAD);
  L.max_pad = std::max(L.n_pad, L.m_pad);
  const size_t B = (size_t)p->batch, n = (size_t)p->n, m = (size_t)p->m, mx = std::max(n, m);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  L.xn = take(8 * B * n);
  L.yn = take(8 * B * m);
  L.la = take(8 * B * n);
  L.lb = take(8 * B * m);
  L.rx = take(8 * B * n);
  L.ry = take(8 * B * m);
  L.maxabs = take(align_up(4 * 2 * B, 16));
  L.qgrid = take(4 * B);
  L.ktag = take(16);  // lambda tags of the two key operands
  // SLACK extra rows after each operand buffer absorb the kernels' unguarded
  // over-reads at the end of the last chunk.
  L.qx = take(2 * (B * L.n_pad + SLACK) * L.KP);
  L.qy = take(2 * (B * L.m_pad + SLACK) * L.KP);
  L.kbx = (L.mode == MODE_SPLIT) ? take(2 * (B * L.n_pad + SLACK) * L.KP) : 0;
  L.kby = (L.mode == MODE_SPLIT) ? take(2 * (B * L.m_pad + SLACK) * L.KP) : 0;
  L.hb = (L.mode == MODE_BF16) ? take(4 * (B * L.max_pad + SLACK)) : 0;
  L.part = take(8 * (size_t)KS_MAX * B * mx);
  L.scratch = take(4 * B * mx);
  L.total = off;
  // Transport: the value operand and the split partials of the P.V pass: room
  // for 16 splits of a one-tile pass, and for the widest pass the partials of
  // 131072 rows (split_rows below, at least one split and at most 16): a few
  // thousand rows of a wide pass need several key splits to fill the GPU.
  const size_t d = (size_t)p->d;
  L.ncols = std::max(p->d <= SK_MAX_D_TRANSPORT ? val_tiles(L.mode, (int)p->d) : 0, apply_tiles(APPLY_COLS)) * 16;
  const size_t split_rows = std::max(B * mx, std::min(16 * B * mx, (size_t)131072));
  L.bpv_bytes = std::max<size_t>(4 * 16 * 16 * B * mx, 4 * split_rows * (size_t)L.ncols);
  L.vt = take(2 * B * (size_t)L.max_pad * L.ncols);
  L.bpv = take(L.bpv_bytes);
  L.bs = take(4 * 16 * B * mx);
  L.bm = take(4 * 16 * B * mx);  // per-split row offsets of the lazy transport pass
  L.ttotal = off;
  // Hessian-vector products: per-row vectors and small matrices, O((n+m) d)
  const size_t bm = B * mx;
  L.h_lse_r = take(4 * bm);
  L.h_lse_k = take(4 * bm);
  L.h_mr = take(8 * bm);
  L.h_mk = take(8 * bm);
  L.h_py = take(4 * bm * d);
  L.h_mat = take(4 * bm * std::max<size_t>(d + 2, std::max<size_t>((size_t)APPLY_COLS, d)));
  L.h_w = take(4 * bm * (d + 2));
  L.h_g = take(4 * bm * (d + 1));
  L.h_quad = take(8 * bm * d);
  L.h_u = take(2 * 2 * (B * (size_t)L.max_pad + SLACK) * L.KP);  // two query-layout planes of the direction
  L.h_zr = take(8 * bm);
  L.h_cr = take(8 * bm);
  L.h_rhs = take(8 * bm);
  L.h_dg = take(8 * bm);
  L.h_res = take(8 * bm);
  L.h_pd = take(8 * bm);
  L.h_pdf = take(4 * bm);
  L.h_t = take(4 * bm);
  L.h_q = take(4 * bm);
  L.h_st = take(8 * 8 * (size_t)B);
  L.h_part = take(8 * 3 * (size_t)B * ((mx + CG_BLK - 1) / CG_BLK));
  L.htotal = off;
  return L;
}

using LseFn = void (*)(const u16*, const u16*, const float*, const float*, const double*, float*, float2*, int, int,
                       int, int, int, int, float, double, unsigned*, unsigned);

template <int MODE, int NCH>
LseFn lse_fn() {
  if constexpr ((MODE == MODE_SPLIT && NCH <= MAX_NCH_SPLIT) || (MODE == MODE_BF16 && NCH <= MAX_NCH_BF16))
    return &k_lse<MODE, NCH>;
  else
    return nullptr;
}

template <int MODE, int... N>
LseFn lse_lookup_impl(int nch, std::integer_sequence<int, N...>) {
  LseFn fn = nullptr;
  ((nch == N + 1 ? (fn = lse_fn<MODE, N + 1>(), 0) : 0), ...);
  return fn;
}

template <int MODE>
LseFn lse_lookup(int nch) {
  constexpr int MAXN = MODE == MODE_SPLIT ? MAX_NCH_SPLIT : MAX_NCH_BF16;
  return lse_lookup_impl<MODE>(nch, std::make_integer_sequence<int, MAXN>{});
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
sk_status resident_capacity(const void* fn, int* out, int block = 256) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    set_err("hipGetDevice failed");
    return SK_EHIP;
  }
  const auto key = std::make_pair(dev, fn);
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(key);
  if (it != cache.end()) {
    *out = it->second;
    return SK_OK;
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, block, 0) !=
          hipSuccess) {
    set_err("occupancy query failed");
    return SK_EHIP;
  }
  *out = cache[key] = std::max(1, cus * std::max(1, per_cu));
  return SK_OK;
}

// Number of key splits ks (and chunks per split) for `rowgroups` row-block
// workgroups: every split does nearly the same work, and rowgroups*ks is chosen
// to fill whole waves of the `capacity` resident slots, so no round of
// workgroups runs nearly empty at the end of the kernel.
int choose_key_splits(int rowgroups, int total_chunks, int capacity, int* cps_out, int ks_cap = KS_MAX) {
  const int kmax = std::max(1, std::min(ks_cap, total_chunks / 2));
  // busy fraction of the resident slots x balance of the split sizes; the
  // fewest splits within 2% of the best (each split adds merge traffic)
  auto score = [&](int ks) {
    const int cps = (total_chunks + ks - 1) / ks;
    const int ks_eff = (total_chunks + cps - 1) / cps;
    const double wgs = (double)rowgroups * ks_eff;
    const double rounds = std::ceil(wgs / capacity);
    return (wgs / (rounds * capacity)) * ((double)total_chunks / ((double)ks_eff * cps));
  };
  double best_score = 0.0;
  for (int ks = 1; ks <= kmax; ++ks) best_score = std::max(best_score, score(ks));
  int best = kmax;
  for (int ks = 1; ks <= kmax; ++ks)
    if (score(ks) >= 0.98 * best_score) {
      best = ks;
      break;
    }
  const int cps = (total_chunks + best - 1) / best;
  *cps_out = cps;
  return (total_chunks + cps - 1) / cps;
}

bool eps_ok(float eps) { return eps > 0.f && isfinite(eps) && isfinite((float)(LOG2E / eps)); }

// Key operand of one side for the potential pot_in and eps: the split key rows
// (fp32 path) or the half bias (bf16 path).  Returns the key operand and bias.
sk_status prep_keys(const sk_problem* p, const void* X, const void* Y, char* w, const Layout& L, const float* pot_in,
                    float eps, int side, hipStream_t stream, const u16** Kop, const float** hb,
                    unsigned** tag_out = nullptr) {
  const int B = (int)p->batch;
  const int keys = (int)(side == 0 ? p->m : p->n);
  const int keys_pad = side == 0 ? L.m_pad : L.n_pad;
  const double* knorm = reinterpret_cast<const double*>(w + (side == 0 ? L.yn : L.xn));
  const double* klogw = reinterpret_cast<const double*>(w + (side == 0 ? L.lb : L.la));
  const float* maxabs = reinterpret_cast<const float*>(w + L.maxabs);
  float* qgrid = reinterpret_cast<float*>(w + L.qgrid);
  const void* Kraw = side == 0 ? Y : X;
  const float lam = (float)(LOG2E / (double)eps);
  *hb = nullptr;
  if (L.mode == MODE_SPLIT) {
    u16* kb = reinterpret_cast<u16*>(w + L.kb(side));
    unsigned* tag = reinterpret_cast<unsigned*>(w + L.ktag) + side;
    // about PREP_SEGS segments per thread when every segment is rebuilt
    const dim3 kgrid((unsigned)(((long long)keys_pad * (L.KP / 8) + 256 * PREP_SEGS - 1) / (256 * PREP_SEGS)), B);
    const double* krn = reinterpret_cast<const double*>(w + (side == 0 ? L.ry : L.rx));
    hipLaunchKernelGGL(k_prep_keys, kgrid, dim3(256), 0, stream, Kraw, L.in_bf16, krn, pot_in, knorm,
                       klogw, keys, keys_pad, (int)p->d, L.KP, lam, eps, maxabs + (side == 0 ? 0 : B),
                       maxabs + (side == 0 ? B : 0), qgrid, tag, kb);
    *Kop = kb;
    if (tag_out != nullptr) *tag_out = tag;
  } else {
    float* hbw = reinterpret_cast<float*>(w + L.hb);
    const dim3 pgrid((keys_pad + 255) / 256, B);
    hipLaunchKernelGGL(k_prep_bias, pgrid, dim3(256), 0, stream, pot_in, knorm, klogw, keys, keys_pad, eps, hbw);
    *hb = hbw;
    *Kop = reinterpret_cast<const u16*>(w + (side == 0 ? L.qy : L.qx));
  }
  return hip_check("key preparation launch");
}

// One half-step.  side 0: f from g (queries X, keys Y); side 1: g from f.
sk_status half_step(const sk_problem* p, const void* X, const void* Y, void* ws, const Layout& L,
                    const float* pot_in, float eps, float* pot_out, int side, hipStream_t stream) {
  char* w = static_cast<char*>(ws);
  const int B = (int)p->batch;
  const int rows = (int)(side == 0 ? p->n : p->m);
  const int keys = (int)(side == 0 ? p->m : p->n);
  const int rows_pad = side == 0 ? L.n_pad : L.m_pad;
  const int keys_pad = side == 0 ? L.m_pad : L.n_pad;
  const double* qnorm = reinterpret_cast<const double*>(w + (side == 0 ? L.xn : L.yn));
  const float* qgrid = reinterpret_cast<const float*>(w + L.qgrid);
  const u16* Qop = reinterpret_cast<const u16*>(w + (side == 0 ? L.qx : L.qy));
  const int nch = L.KP / 32;
  const int cfMW = cfg_MW(L.mode, nch), cfR = cfg_R(L.mode, nch), cfTC = cfg_TC(L.mode, nch);
  const float lam = (float)(LOG2E / (double)eps);

  const u16* Kop = nullptr;
  const float* hb = nullptr;
  unsigned* tag = nullptr;
  sk_status st = prep_keys(p, X, Y, w, L, pot_in, eps, side, stream, &Kop, &hb, &tag);
  if (st != SK_OK) return st;

  LseFn fn = (L.mode == MODE_SPLIT) ? lse_lookup<MODE_SPLIT>(nch) : lse_lookup<MODE_BF16>(nch);
  int tc = cfTC;
  if (L.mode == MODE_SPLIT && nch == 1 && keys < SMALL_KEYS) {
    // fewer keys than a few workgroups' worth of 256-key chunks: 128-key chunks fill the GPU better
    fn = &k_lse<MODE_SPLIT, 1, SMALL_TC>;
    tc = SMALL_TC;
  }
  if (fn == nullptr) {
    set_err("no kernel for %d K chunks", nch);
    return SK_EUNSUPPORTED;
  }
  const int NW = cfg_NW(L.mode, nch);
  const int wg_x = (rows + NW * cfR * cfMW - 1) / (NW * cfR * cfMW);
  const int CK = tc * cfMW;
  const int total_chunks = (keys + CK - 1) / CK;
  int capacity = 0;
  st = resident_capacity(reinterpret_cast<const void*>(fn), &capacity, 64 * NW);
  if (st != SK_OK) return st;
  int cps = 0;
  const int ks = choose_key_splits(wg_x * B, total_chunks, capacity, &cps);
  float2* part = ks > 1 ? reinterpret_cast<float2*>(w + L.part) : nullptr;
  const double inv_lam = 1.0 / (double)lam;
  hipLaunchKernelGGL(fn, dim3(wg_x, ks, B), dim3(64 * NW), 0, stream, Qop, Kop, hb, qgrid, qnorm, pot_out, part, rows,
                     rows_pad, keys, keys_pad, cps, B, 2.f * lam, inv_lam, tag, __builtin_bit_cast(unsigned, lam));
  st = hip_check("half-step kernel launch");
  if (st != SK_OK || ks == 1) return st;
  const int total = B * rows;
  hipLaunchKernelGGL(k_merge, dim3((total + 255) / 256), dim3(256), 0, stream, part, ks, total, qnorm, pot_out,
                     inv_lam);
  return hip_check("split merge launch");
}

using BaryFn = void (*)(const u16*, const u16*, const float*, const u16*, const float*, const double*, const float*,
                        float*, float*, int, int, int, int, int, int, float, float, float*, unsigned*, unsigned,
                        const u16*, float);

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
  if (mode == MODE_SPLIT) return bary_lookup_impl<MODE_SPLIT>(d, std::make_integer_sequence<int, SK_MAX_D_FP32>{});
  return bary_lookup_impl<MODE_BF16>(d, std::make_integer_sequence<int, SK_MAX_D_TRANSPORT>{});
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
  const float* qgrid = reinterpret_cast<const float*>(w + L.qgrid);
  const u16* Qop = reinterpret_cast<const u16*>(w + (side == 0 ? L.qx : L.qy));
  const void* Praw = side == 0 ? X : Y;
  const void* Kraw = side == 0 ? Y : X;
  const float* pot_row = side == 0 ? f : g;
  float* lse = reinterpret_cast<float*>(w + L.scratch);

  // 1. The key operand of this side for the other potential and eps.  The P.V
  //    pass keeps lazy row offsets, so no half-step runs first: its merge
  //    recovers each row's log-sum-exp (into scratch) from the offsets and sums.
  const u16* Kop = nullptr;
  const float* hb = nullptr;
  unsigned* tag = nullptr;
  sk_status st = prep_keys(p, X, Y, w, L, side == 0 ? g : f, eps, side, stream, &Kop, &hb, &tag);
  if (st != SK_OK) return st;

  // 2. Value operand from the other cloud's coordinates.
  u16* vt = reinterpret_cast<u16*>(w + L.vt);
  const int nc = val_tiles(L.mode, d) * 16;
  const long long nvec = (long long)(keys_pad / VK) * nc * (VK / 8);
  const int sumcol = val_sumcol(L.mode, d) ? 1 : 0;
  const double* krn = reinterpret_cast<const double*>(w + (side == 0 ? L.ry : L.rx));
  hipLaunchKernelGGL(k_prep_vals, dim3((unsigned)((nvec + 255) / 256), B), dim3(256), 0, stream, Kraw, L.mode,
                     L.in_bf16, krn, keys, keys_pad, d, nc, sumcol, vt);
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
  hipLaunchKernelGGL(fn, dim3(wg_x, ks, B), dim3(64 * NWb), 0, stream, Qop, Kop, hb, vt, qgrid, qnorm, nullptr, bpv, bs, rows,
                     rows_pad, keys, keys_pad, cps, B, lam, 2.f * lam, bm, tag, __builtin_bit_cast(unsigned, lam), nullptr,
                     1.f);
  st = hip_check("transport kernel launch");
  if (st != SK_OK) return st;

  // 4. Merge the splits, divide, form the gradient.
  const long long total = (long long)B * rows * d;
  hipLaunchKernelGGL(k_bary_merge, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, bpv, bs, ks, B, rows,
                     d, nc, val_parts(L.mode), sumcol, Praw, L.in_bf16, pot_row, lse, qlogw, (double)eps, bm, qnorm,
                     1.0 / (double)lam, bary, L.cosine ? nullptr : grad);
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
    return apply_lookup_impl<MODE_SPLIT>(d, nct, std::make_integer_sequence<int, SK_MAX_D_FP32>{});
  return apply_lookup_impl<MODE_BF16>(d, nct, std::make_integer_sequence<int, SK_MAX_D_TRANSPORT>{});
}

// out[b][row][k] = sum_j P_ij M[b][j][k] (k < c) for one side (side 0: rows are
// the points of X, keys those of Y), at potentials pot_row / pot_key whose
// half-step values for the rows are lse.  Columns go in passes of APPLY_COLS.
sk_status apply_plan(const sk_problem* p, const void* X, const void* Y, char* w, const Layout& L,
                     const float* pot_row, const float* pot_key, const float* lse, float eps, int side,
                     const float* M, int c, float* out, hipStream_t stream) {
  const int B = (int)p->batch, d = (int)p->d;
  const int rows = (int)(side == 0 ? p->n : p->m);
  const int keys = (int)(side == 0 ? p->m : p->n);
  const int rows_pad = side == 0 ? L.n_pad : L.m_pad;
  const int keys_pad = side == 0 ? L.m_pad : L.n_pad;
  const double* qnorm = reinterpret_cast<const double*>(w + (side == 0 ? L.xn : L.yn));
  const double* qlogw = reinterpret_cast<const double*>(w + (side == 0 ? L.la : L.lb));
  const float* qgrid = reinterpret_cast<const float*>(w + L.qgrid);
  const u16* Qop = reinterpret_cast<const u16*>(w + (side == 0 ? L.qx : L.qy));
  const u16* Kop = nullptr;
  const float* hb = nullptr;
  unsigned* ptag = nullptr;
  sk_status st = prep_keys(p, X, Y, w, L, pot_key, eps, side, stream, &Kop, &hb, &ptag);
  if (st != SK_OK) return st;
  u16* vt = reinterpret_cast<u16*>(w + L.vt);
  float* bpv = reinterpret_cast<float*>(w + L.bpv);
  float* bs = reinterpret_cast<float*>(w + L.bs);
  const float lam = (float)(LOG2E / (double)eps);
  const int nch = L.KP / 32;
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
    hipLaunchKernelGGL(fn, dim3(wg_x, ks, B), dim3(64 * NWb), 0, stream, Qop, Kop, hb, vt, qgrid, qnorm, lse, bpv, bs,
                       rows, rows_pad, keys, keys_pad, cps, B, lam, 2.f * lam, nullptr, ptag,
                       __builtin_bit_cast(unsigned, lam), nullptr, 1.f);
    st = hip_check("plan-application kernel launch");
    if (st != SK_OK) return st;
    const long long total = (long long)B * rows * cb;
    hipLaunchKernelGGL(k_apply_merge, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, bpv, ks, B, rows,
                       cb, nc, c, col0, qlogw, pot_row, lse, (double)eps, out);
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
  if (mode == MODE_SPLIT) return uw_lookup_impl<MODE_SPLIT>(d, std::make_integer_sequence<int, SK_MAX_D_FP32>{});
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
  const float* qgrid = reinterpret_cast<const float*>(w + L.qgrid);
  const u16* Qop = reinterpret_cast<const u16*>(w + (side == 0 ? L.qx : L.qy));
  const void* Kraw = side == 0 ? Y : X;
  const u16* Kop = nullptr;
  const float* hb = nullptr;
  unsigned* ptag = nullptr;
  sk_status st = prep_keys(p, X, Y, w, L, pot_key, eps, side, stream, &Kop, &hb, &ptag);
  if (st != SK_OK) return st;
  u16* U = reinterpret_cast<u16*>(w + L.h_u);
  hipLaunchKernelGGL(k_prep_u, dim3((rows_pad + 255) / 256, B), dim3(256), 0, stream, Vdir, rows, rows_pad, d, L.KP,
                     L.mode, B, U);
  u16* vt = reinterpret_cast<u16*>(w + L.vt);
  const int nct = val_tiles(L.mode, d), nc = nct * 16;
  const long long nvec = (long long)(keys_pad / VK) * nc * (VK / 8);
  const double* krn = reinterpret_cast<const double*>(w + (side == 0 ? L.ry : L.rx));
  hipLaunchKernelGGL(k_prep_vals, dim3((unsigned)((nvec + 255) / 256), B), dim3(256), 0, stream, Kraw, L.mode,
                     L.in_bf16, krn, keys, keys_pad, d, nc, 0, vt);
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
  hipLaunchKernelGGL(fn, dim3(wg_x, ks, B), dim3(64 * NWb), 0, stream, Qop, Kop, hb, vt, qgrid, qnorm, lse, bpv, bs, rows,
                     rows_pad, keys, keys_pad, cps, B, lam, 2.f * lam, nullptr, ptag, __builtin_bit_cast(unsigned, lam),
                     U, ugain);
  st = hip_check("row-weighted plan kernel launch");
  if (st != SK_OK) return st;
  const long long total = (long long)B * rows * d;
  hipLaunchKernelGGL(k_uw_merge, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, bpv, bs, ks, B, rows, d,
                     nc, val_parts(L.mode), qlogw, pot_row, lse, (double)eps, quad);
  return hip_check("row-weighted merge launch");
}

unsigned blocks_for(long long n) { return (unsigned)((n + 255) / 256); }

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
  hipLaunchKernelGGL(k_coords, dim3(blocks_for(nk * d)), dim3(256), 0, s, Qraw, in16, nk * d, mat);
  st = hip_check("HVP set-up launch");
  if (st == SK_OK) st = apply_plan(p, X, Y, w, L, pot_r, pot_k, lse_r, eps, side, mat, d, py, s);
  if (st != SK_OK) return st;
  // 3. right-hand side: cr per moving row, then P^T [z, v, cr/r] per fixed row
  hipLaunchKernelGGL(k_hvp_rows, dim3(blocks_for(nr)), dim3(256), 0, s, Praw, in16, V, py, mr, nr, d, zr, cr, mat);
  st = hip_check("HVP rows launch");
  if (st == SK_OK) st = apply_plan(p, X, Y, w, L, pot_k, pot_r, lse_k, eps, 1 - side, mat, d + 2, wk, s);
  if (st != SK_OK) return st;
  hipLaunchKernelGGL(k_hvp_rhs, dim3(blocks_for(nk)), dim3(256), 0, s, Qraw, in16, wk, nk, d, rhs);
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
  for (int64_t it = 0; it < cg_iters; ++it) {
    st = apply_plan(p, X, Y, w, L, pot_r, pot_k, lse_r, eps, side, pdf, 1, tv, s);
    if (st != SK_OK) return st;
    hipLaunchKernelGGL(k_div_mass, dim3(blocks_for(nr)), dim3(256), 0, s, tv, mr, nr);
    st = apply_plan(p, X, Y, w, L, pot_k, pot_r, lse_k, eps, 1 - side, tv, 1, qv, s);
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
  hipLaunchKernelGGL(k_hvp_gmat, dim3(blocks_for(nk)), dim3(256), 0, s, Qraw, in16, dg, nk, d, mat);
  st = hip_check("HVP matrix launch");
  if (st == SK_OK) st = apply_plan(p, X, Y, w, L, pot_r, pot_k, lse_r, eps, side, mat, d + 1, gm, s);
  if (st != SK_OK) return st;
  // 6. sum_j P_ij (q_j . v_i) q_j = M_i v_i in one row-weighted plan pass
  st = apply_uw(p, X, Y, w, L, pot_r, pot_k, lse_r, eps, side, V, quad, s);
  if (st != SK_OK) return st;
  // 7. assemble
  hipLaunchKernelGGL(k_hvp_final, dim3(blocks_for(nr)), dim3(256), 0, s, Praw, in16, V, py, mr, zr, cr, gm, quad, nr,
                     d, (double)eps, out);
  return hip_check("HVP assembly launch");
}

sk_status init_impl(const sk_problem* p, const void* X, const void* Y, const float* a, const float* b, void* ws,
                    const Layout& L, hipStream_t stream) {
  char* w = static_cast<char*>(ws);
  const int B = (int)p->batch;
  float* maxabs = reinterpret_cast<float*>(w + L.maxabs);
  auto zero = [&](size_t off, size_t bytes) {
    const size_t n16 = bytes / 16;
    if (n16) hipLaunchKernelGGL(k_zero, dim3((unsigned)std::min<size_t>((n16 + 255) / 256, 4096)), dim3(256), 0,
                                stream, reinterpret_cast<u4*>(w + off), n16);
  };
  if (L.cosine) {
    // normalised points: every coordinate is at most 1 in magnitude
    hipLaunchKernelGGL(k_fill_f32, dim3((2 * B + 255) / 256), dim3(256), 0, stream, maxabs, 2 * B, 1.f);
  } else {
    zero(L.maxabs, align_up(8 * (size_t)B, 16));
    const long long most = std::max(p->n, p->m) * p->d;
    const unsigned mblocks = (unsigned)std::min<long long>((most + 255) / 256, 64);
    hipLaunchKernelGGL(k_maxabs, dim3(mblocks, B, 2), dim3(256), 0, stream, X, Y, L.in_bf16,
                       (long long)(p->n * p->d), (long long)(p->m * p->d), reinterpret_cast<unsigned*>(maxabs), B);
  }
  auto side = [&](const void* P, const float* wt, int rows, int rows_pad, const float* mabs, size_t norm,
                  size_t logw, size_t rnorm, size_t op) {
    const dim3 grid((rows_pad + 255) / 256, B);
    if (L.mode == MODE_SPLIT)
      hipLaunchKernelGGL(k_init_side<MODE_SPLIT>, grid, dim3(256), 0, stream, P, wt, rows, rows_pad, (int)p->d,
                         L.KP, L.in_bf16, L.cosine, mabs, reinterpret_cast<double*>(w + norm),
                         reinterpret_cast<double*>(w + logw), reinterpret_cast<double*>(w + rnorm),
                         reinterpret_cast<u16*>(w + op));
    else
      hipLaunchKernelGGL(k_init_side<MODE_BF16>, grid, dim3(256), 0, stream, P, wt, rows, rows_pad, (int)p->d,
                         L.KP, L.in_bf16, L.cosine, mabs, reinterpret_cast<double*>(w + norm),
                         reinterpret_cast<double*>(w + logw), reinterpret_cast<double*>(w + rnorm),
                         reinterpret_cast<u16*>(w + op));
  };
  side(X, a, (int)p->n, L.n_pad, maxabs, L.xn, L.la, L.rx, L.qx);
  side(Y, b, (int)p->m, L.m_pad, maxabs + B, L.yn, L.lb, L.ry, L.qy);
  // the slack rows after the last problem's operand rows: a workgroup whose
  // query rows run past the padding reads zeros there
  zero(L.qx + 2 * (size_t)B * L.n_pad * L.KP, 2 * (size_t)SLACK * L.KP);
  zero(L.qy + 2 * (size_t)B * L.m_pad * L.KP, 2 * (size_t)SLACK * L.KP);
  // new clouds: the key operands hold no coordinate parts yet
  if (L.mode == MODE_SPLIT) zero(L.ktag, 16);
  return hip_check("init kernel launch");
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
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = init_impl(p, X, Y, a, b, ws, L, s);
  for (int64_t k = 0; k < iters && st == SK_OK; ++k) {
    const float e = eps[n_eps == 1 ? 0 : k];
    st = half_step(p, X, Y, ws, L, g, e, f, 0, s);
    if (st == SK_OK) st = half_step(p, X, Y, ws, L, f, e, g, 1, s);
  }
  return st;
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

// Transport, plan products and HVPs keep the query operand of the P.V kernel in
// registers: d <= SK_MAX_D_TRANSPORT.
static sk_status check_transport_d(const sk_problem* p) {
  if (p->d > SK_MAX_D_TRANSPORT) {
    set_err("d = %lld exceeds SK_MAX_D_TRANSPORT = %d for transport, plan and HVP calls", (long long)p->d,
            SK_MAX_D_TRANSPORT);
    return SK_EUNSUPPORTED;
  }
  return SK_OK;
}

static sk_status transport_entry(const sk_problem* p, const void* X, const void* Y, void* ws, size_t ws_bytes,
                                 const float* f, const float* g, float eps, float* bary, float* grad, void* stream,
                                 int side) {
  g_err[0] = 0;
  Layout L;
  sk_status st = check_ws(p, ws, ws_bytes, &L, 1);
  if (st == SK_OK) st = check_transport_d(p);
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
  if (st == SK_OK) st = check_transport_d(p);
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
  if (st == SK_OK) st = check_transport_d(p);
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
