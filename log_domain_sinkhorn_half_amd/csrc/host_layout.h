// Host-side layout and validation of the log-domain Sinkhorn library:
// constants shared with the kernels, the workspace layout, the argument checks
// and the choice of key splits.  Pure host arithmetic (no HIP calls), so the
// same text is compiled into the library and into a host-only sanitizer build.
//
// This is a fragment: it is included inside an unnamed namespace, after
// <algorithm>, <math.h>, <stdarg.h>, <stdint.h> and "sinkhorn.h", with SK_HD
// defined as the function qualifiers for host and device (empty on the host),
// and with set_err (printf-style, sets the text sinkhorn_last_error returns)
// defined by the including translation unit.

void set_err(const char* fmt, ...) __attribute__((format(printf, 1, 2)));

constexpr int MODE_SPLIT = 0;  // fp32 inputs
constexpr int MODE_BF16 = 1;   // bf16 inputs
constexpr int MODE_HILO = 2;   // fp32 inputs wider than SK_MAX_D_SPLIT: hi/lo operands, K loop
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
// At most this many scores per problem (rows x keys) the d <= 3 half-step runs
// TINY_R query tiles per wave, TINY_TC key tiles per chunk and no key split.
constexpr long long TINY_WORK = 1LL << 21;
constexpr int TINY_R = 1;
constexpr int TINY_TC = 8;
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
SK_HD constexpr int split_grid_slots(int d) { return d + 5; }
SK_HD constexpr int split_corr_slots(int d) { return 7 * d + 2; }
SK_HD constexpr bool split_single(int d) { return split_grid_slots(d) <= 8 && split_corr_slots(d) <= 24; }
SK_HD constexpr int split_corr_begin(int d) {
  return split_single(d) ? 8 : (split_grid_slots(d) + 31) / 32 * 32;
}
SK_HD constexpr int split_nch(int d) {
  return split_single(d) ? 1 : (split_corr_begin(d) + split_corr_slots(d) + 31) / 32;
}
constexpr int MAX_NCH_SPLIT = split_nch(SK_MAX_D_SPLIT);
constexpr int MAX_NCH_BF16 = (SK_MAX_D + 31) / 32;

// ---------------------------------------------------------------------------
// Value operand of the transport and plan passes (per 32-key block)
// ---------------------------------------------------------------------------
constexpr int VK = 32;  // keys per value block: one 16x16x32 K step, two 16-key score tiles

// bf16 parts of a coordinate in the value operand: three hold an fp32 value
// exactly (split path), two hold 16 significant bits (hi/lo path), and bf16
// inputs are exact in one.
SK_HD constexpr int val_parts(int mode) { return mode == MODE_SPLIT ? 3 : (mode == MODE_HILO ? 2 : 1); }
SK_HD constexpr int val_tiles(int mode, int d) { return (val_parts(mode) * d + 15) / 16; }
// A spare value column holds ones, so the P.V product also yields the sum of the weights.
SK_HD constexpr bool val_sumcol(int mode, int d) { return val_parts(mode) * d < val_tiles(mode, d) * 16; }

constexpr int APPLY_COLS = 64;  // matrix columns per pass (3 parts each + the ones column <= 13 tiles)

SK_HD constexpr int apply_tiles(int cb) { return cb <= 5 ? 1 : (cb <= 21 ? 4 : 13); }

// Wide plan passes (hi/lo operands, or bf16 operands past SK_MAX_D_TRANSPORT)
// go through a weights buffer of one block of rows against all keys, at most
// this many bytes (the block shrinks to fit, down to 256 rows).
constexpr size_t WIDE_WT_BYTES = (size_t)1 << 30;

// Conjugate-gradient vectors are reduced in blocks of this many elements.
constexpr int CG_BLK = 2048;

// ---------------------------------------------------------------------------
// Workspace layout and argument checks
// ---------------------------------------------------------------------------
struct Layout {
  int mode, KP, n_pad, m_pad, max_pad;
  int in_bf16, cosine;
  size_t xn, yn, la, lb, rx, ry, maxabs, cen, box, inexact, status, qgrid, ktag, qx, qy, kbx, kby, hb, hb1, part,
      scratch, total;
  size_t hbs(int side) const { return side == 0 ? hb : hb1; }
  // key operand of the fp32 path for side 0 (Y as keys) or side 1 (X as keys)
  size_t kb(int side) const { return side == 0 ? kby : kbx; }
  // transport application and plan products (after `total`; only their entry points need them)
  int ncols;             // widest value operand (columns) of any transport pass
  bool wide;             // plan passes through the weights buffer
  int wt_rows;           // rows per block of the weights buffer (wide)
  int wide_cols;         // matrix columns per wide plan-application pass (3 parts each)
  size_t wt;             // weights buffer (wide)
  size_t bpv_bytes;      // bytes of the split-partials region
  size_t vt, bpv, bs, bm, ttotal;
  // Hessian-vector products (after `ttotal`)
  size_t h_lse_r, h_lse_k, h_mr, h_mk, h_py, h_mat, h_w, h_g, h_quad, h_zr, h_cr, h_rhs, h_dg, h_res,
      h_pd, h_pdf, h_t, h_q, h_st, h_part, h_u, h_wsr, h_wsk, htotal;
};

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int kp_for(int mode, int64_t d) {
  if (mode == MODE_SPLIT) return split_nch((int)d) * 32;
  if (mode == MODE_HILO) return (int)align_up((size_t)(3 * d), 32);  // (x_h, x_h, x_l) per coordinate
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
  if (p->dtype == SK_FP32 && p->d > SK_MAX_D_FP32) {
    set_err("d = %lld exceeds SK_MAX_D_FP32 = %d for fp32 inputs", (long long)p->d, SK_MAX_D_FP32);
    return SK_EUNSUPPORTED;
  }
  if (p->cost == SK_COST_COSINE && p->d > SK_MAX_D_SPLIT) {
    set_err("d = %lld exceeds SK_MAX_D_SPLIT = %d for the cosine cost", (long long)p->d, SK_MAX_D_SPLIT);
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
  // bf16 operands are used as they are; fp32 inputs and normalised points take
  // the split layout, fp32 inputs wider than SK_MAX_D_SPLIT the hi/lo layout
  L.mode = (L.in_bf16 && !L.cosine) ? MODE_BF16 : (p->d > SK_MAX_D_SPLIT ? MODE_HILO : MODE_SPLIT);
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
  L.cen = take(8 * B * (size_t)p->d);               // centre of each problem (fp64)
  L.box = take(4 * 4 * B * (size_t)p->d);           // bounding boxes of both clouds (ordered codes)
  L.inexact = take(4 * B);                          // bf16 problems left uncentred
  L.status = take(16);                              // range flags (SK_FLAG_*)
  L.qgrid = take(4 * 2 * B);  // grid quantum of each side's key operand, [side][B]
  L.ktag = take(16);  // lambda tags of the two key operands
  // SLACK extra rows after each operand buffer absorb the kernels' unguarded
  // over-reads at the end of the last chunk.
  L.qx = take(2 * (B * L.n_pad + SLACK) * L.KP);
  L.qy = take(2 * (B * L.m_pad + SLACK) * L.KP);
  L.kbx = (L.mode != MODE_BF16) ? take(2 * (B * L.n_pad + SLACK) * L.KP) : 0;
  L.kby = (L.mode != MODE_BF16) ? take(2 * (B * L.m_pad + SLACK) * L.KP) : 0;
  // half bias of each side's keys (bf16 path): side 0 (keys Y) then side 1 (keys X)
  L.hb = (L.mode != MODE_SPLIT) ? take(4 * (B * L.m_pad + SLACK)) : 0;
  L.hb1 = (L.mode != MODE_SPLIT) ? take(4 * (B * L.n_pad + SLACK)) : 0;
  L.part = take(8 * (size_t)KS_MAX * B * mx);
  L.scratch = take(4 * B * mx);
  L.total = off;
  // Transport: the value operand and the split partials of the P.V pass: room
  // for 16 splits of a one-tile pass, and for the widest pass the partials of
  // 131072 rows (split_rows below, at least one split and at most 16): a few
  // thousand rows of a wide pass need several key splits to fill the GPU.
  const size_t d = (size_t)p->d;
  L.wide = L.mode == MODE_HILO || (L.mode == MODE_BF16 && p->d > SK_MAX_D_TRANSPORT);
  // keys of a wide pass, rounded up to whole 256-key blocks
  const size_t kcov = align_up(mx, 256);
  if (L.wide) {
    // value columns (the parts of each coordinate) or three parts of wide_cols
    // matrix columns, in whole 256-column blocks of the product
    L.ncols = (int)align_up(std::max<size_t>(val_parts(L.mode) * d, 3 * APPLY_COLS), 256);
    L.wide_cols = L.ncols / 3;
    const size_t per_row = 2 * B * 2 * kcov;  // bytes of one weights row (hi and lo) over the batch
    L.wt_rows = (int)std::min(align_up(mx, 256), std::max<size_t>(256, WIDE_WT_BYTES / per_row / 256 * 256));
  } else {
    L.ncols = std::max(p->d <= SK_MAX_D_TRANSPORT ? val_tiles(L.mode, (int)p->d) : 0, apply_tiles(APPLY_COLS)) * 16;
    L.wide_cols = 0;
    L.wt_rows = 0;
  }
  const size_t split_rows = std::max(B * mx, std::min(16 * B * mx, (size_t)131072));
  // wide passes merge per row block: 16 splits of one block's partials
  const size_t part_rows = std::max(mx, (size_t)L.wt_rows);
  L.bpv_bytes = std::max<size_t>(4 * 16 * 16 * B * mx, 4 * split_rows * (size_t)L.ncols);
  if (L.wide) L.bpv_bytes = std::max(L.bpv_bytes, 4 * 16 * B * (size_t)L.wt_rows * L.ncols);
  // value operand: [B][max_pad / 32][ncols][32] (narrow) or [B][ncols][kcov] (wide)
  L.vt = L.wide ? take(2 * B * (size_t)L.ncols * kcov) : take(2 * B * (size_t)L.max_pad * L.ncols);
  L.wt = L.wide ? take(2 * B * (size_t)L.wt_rows * 2 * kcov) : 0;
  L.bpv = take(L.bpv_bytes);
  L.bs = take(4 * 16 * B * part_rows);
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
  L.h_wsr = take(8 * bm);  // row mass / weight sum of the CG plan passes, moving side
  L.h_wsk = take(8 * bm);  // the same, fixed side
  L.htotal = off;
  return L;
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
