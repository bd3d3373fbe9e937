// Host-only check of the library's layout and validation logic (host_layout.h),
// built with AddressSanitizer and UndefinedBehaviorSanitizer by the CPU test
// suite.  It runs every argument check, the workspace layout and the key-split
// choice over many seeded problems, including the largest accepted sizes, and
// checks their invariants:
//   * invalid problems are rejected with the documented status and a message;
//   * every workspace region starts on a 256-byte boundary, the regions follow
//     one another without overlap, and the three workspace sizes are nested
//     (solver <= transport <= HVP) and grow linearly in the point counts;
//   * key splits cover every key chunk exactly once, within the split cap.
// Prints one summary line; exit status 0 when every check holds.
#include <algorithm>
#include <math.h>
#include <random>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
#include <vector>

#include "sinkhorn.h"

#define SK_HD

namespace {

#include "host_layout.h"

char g_err[512];
void set_err(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

int failures = 0;
long checks = 0;
void expect(bool ok, const char* what, const sk_problem& p) {
  ++checks;
  if (!ok && failures++ < 20)
    fprintf(stderr, "FAILED %s for batch=%lld n=%lld m=%lld d=%lld dtype=%d cost=%d\n", what, (long long)p.batch,
            (long long)p.n, (long long)p.m, (long long)p.d, p.dtype, p.cost);
}

// Regions in the order layout_of takes them, with a lower bound on each size.
void check_layout(const sk_problem& p) {
  const Layout L = layout_of(&p);
  const size_t B = (size_t)p.batch, n = (size_t)p.n, m = (size_t)p.m, d = (size_t)p.d;
  const size_t mx = std::max(n, m);
  struct R {
    size_t off, min_bytes;
  };
  std::vector<R> regs = {{L.xn, 8 * B * n},  {L.yn, 8 * B * m},      {L.la, 8 * B * n},        {L.lb, 8 * B * m},
                         {L.rx, 8 * B * n},  {L.ry, 8 * B * m},      {L.maxabs, 8 * B},        {L.cen, 8 * B * d},
                         {L.box, 16 * B * d}, {L.inexact, 4 * B},   {L.status, 4},            {L.qgrid, 8 * B},
                         {L.ktag, 16},       {L.qx, 2 * B * n * (size_t)L.KP}, {L.qy, 2 * B * m * (size_t)L.KP}};
  if (L.mode != MODE_BF16) {
    regs.push_back({L.kbx, 2 * B * n * (size_t)L.KP});
    regs.push_back({L.kby, 2 * B * m * (size_t)L.KP});
  }
  if (L.mode != MODE_SPLIT) {
    regs.push_back({L.hb, 4 * B * m});
    regs.push_back({L.hb1, 4 * B * n});
  }
  regs.push_back({L.part, 8 * (size_t)KS_MAX * B * mx});
  regs.push_back({L.scratch, 4 * B * mx});
  bool aligned = true, ordered = true;
  for (size_t k = 0; k < regs.size(); ++k) {
    aligned &= regs[k].off % 256 == 0;
    const size_t end = regs[k].off + regs[k].min_bytes;
    const size_t next = k + 1 < regs.size() ? regs[k + 1].off : L.total;
    ordered &= end <= next;
  }
  expect(aligned, "256-byte alignment of the workspace regions", p);
  expect(ordered, "workspace regions in order without overlap", p);
  // transport regions, between total and ttotal
  const size_t kcov = align_up(mx, 256);
  std::vector<R> tregs;
  tregs.push_back({L.vt, L.wide ? 2 * B * (size_t)L.ncols * kcov : 2 * B * (size_t)L.max_pad * L.ncols});
  if (L.wide) tregs.push_back({L.wt, 2 * B * (size_t)L.wt_rows * 2 * kcov});
  tregs.push_back({L.bpv, std::max<size_t>(L.bpv_bytes, 4 * B * (L.wide ? 16 * (size_t)L.wt_rows : mx) * L.ncols)});
  tregs.push_back({L.bs, 4 * 16 * B * std::max(mx, (size_t)L.wt_rows)});
  tregs.push_back({L.bm, 4 * 16 * B * mx});
  bool tordered = tregs[0].off >= L.total;
  for (size_t k = 0; k < tregs.size(); ++k) {
    const size_t next = k + 1 < tregs.size() ? tregs[k + 1].off : L.ttotal;
    tordered &= tregs[k].off % 256 == 0 && tregs[k].off + tregs[k].min_bytes <= next;
  }
  expect(tordered, "transport regions aligned, in order, without overlap", p);
  expect(!L.wide || (L.ncols % 256 == 0 && L.ncols >= val_parts(L.mode) * (int)d && 3 * L.wide_cols <= L.ncols &&
                     L.wide_cols >= APPLY_COLS),
         "wide value columns: whole 256-column blocks holding the parts", p);
  expect(L.wide == (L.mode == MODE_HILO || (L.mode == MODE_BF16 && p.d > SK_MAX_D_TRANSPORT)),
         "wide passes exactly past the register-resident widths", p);
  expect(L.total <= L.ttotal && L.ttotal <= L.htotal, "nested workspace sizes", p);
  expect(L.n_pad % ROW_PAD == 0 && L.m_pad % ROW_PAD == 0 && L.n_pad >= p.n && L.m_pad >= p.m, "row padding", p);
  const int min_slots = L.mode == MODE_SPLIT ? 8 * (int)d + 7 : (L.mode == MODE_HILO ? 3 * (int)d : (int)d);
  expect(L.KP % 32 == 0 && L.KP >= min_slots, "operand slots", p);
  expect((L.mode == MODE_HILO) == (p.dtype == SK_FP32 && p.cost == SK_COST_SQEUCLID && p.d > SK_MAX_D_SPLIT),
         "hi/lo layout exactly for wide fp32 inputs", p);
  expect(L.mode != MODE_HILO || L.KP >= 2 * 32, "hi/lo operands span at least two K chunks", p);
}

void check_linear(sk_problem p) {
  const Layout L0 = layout_of(&p);
  const size_t a = L0.htotal;
  p.n *= 2;
  p.m *= 2;
  const Layout L1 = layout_of(&p);
  const size_t b = L1.htotal;
  // linear, apart from the wide passes' weights buffer (rows x keys, capped)
  expect(b <= 2 * a + (1u << 24) + (L1.wide ? WIDE_WT_BYTES : 0), "workspace linear in the point counts", p);
  const size_t kcov = align_up((size_t)std::max(p.n, p.m), 256);
  const size_t row_bytes = 2 * (size_t)p.batch * 2 * kcov;
  expect(!L1.wide || (L1.wt_rows % 256 == 0 && L1.wt_rows >= 256 &&
                      (size_t)L1.wt_rows * row_bytes <= std::max(WIDE_WT_BYTES, 256 * row_bytes) &&
                      (size_t)L1.wt_rows <= align_up((size_t)std::max(p.n, p.m), 256)),
         "weights buffer: whole 256-row blocks within its byte cap", p);
}

}  // namespace

int main() {
  std::mt19937_64 rng(12345);
  auto pick = [&](int64_t lo, int64_t hi) { return std::uniform_int_distribution<int64_t>(lo, hi)(rng); };

  // rejected problems
  const sk_problem bad[] = {{0, 5, 5, 3, 0, 0},   {1, 0, 5, 3, 0, 0},    {1, 5, -1, 3, 0, 0}, {1, 5, 5, 0, 0, 0},
                            {1, 5, 5, 1025, 0, 0}, {1, 5, 5, 1025, 1, 0}, {1, 5, 5, 3, 2, 0},  {1, 5, 5, 3, 0, 2},
                            {1, 5, 5, 100, 1, 1}, {65536, 5, 5, 3, 0, 0}, {1, 1LL << 30, 5, 3, 0, 0},
                            {4096, 1 << 20, 5, 3, 0, 0}};
  const sk_status want[] = {SK_ESHAPE, SK_ESHAPE,       SK_ESHAPE,       SK_ESHAPE, SK_EUNSUPPORTED, SK_EUNSUPPORTED,
                            SK_EDTYPE, SK_EINVAL,       SK_EUNSUPPORTED, SK_ESHAPE, SK_ESHAPE,       SK_ESHAPE};
  for (size_t k = 0; k < sizeof(bad) / sizeof(bad[0]); ++k) {
    g_err[0] = 0;
    expect(check_problem(&bad[k]) == want[k] && g_err[0] != 0, "rejection status and message", bad[k]);
  }
  g_err[0] = 0;
  expect(check_problem(nullptr) == SK_EINVAL && g_err[0] != 0, "NULL problem rejected", bad[0]);

  // accepted problems: random shapes, and the largest accepted sizes
  for (int it = 0; it < 20000; ++it) {
    sk_problem p{};
    p.dtype = (int32_t)pick(0, 1);
    p.cost = (int32_t)pick(0, 1);
    const int dmax = p.cost == SK_COST_COSINE ? SK_MAX_D_SPLIT : (p.dtype == SK_FP32 ? SK_MAX_D_FP32 : SK_MAX_D);
    p.d = pick(1, dmax);
    p.batch = pick(1, it % 10 == 0 ? 300 : 4);
    p.n = pick(1, it % 7 == 0 ? 200000 : 5000);
    p.m = pick(1, it % 5 == 0 ? 200000 : 5000);
    if (check_problem(&p) != SK_OK) {
      expect(false, "random valid problem accepted", p);
      continue;
    }
    check_layout(p);
    check_linear(p);
  }
  const sk_problem big[] = {{1, (1LL << 30) - 1, 7, 3, 0, 0},
                            {1, 3, (1LL << 30) - 1, 1024, 1, 0},
                            {2047, (1LL << 20) - 1, 1000, 88, 0, 0},
                            {65535, 32767, 32767, 1, 0, 1}};
  for (const sk_problem& p : big) {
    expect(check_problem(&p) == SK_OK, "largest accepted problem", p);
    check_layout(p);
  }

  // key splits: every chunk covered once, at most the cap
  for (int it = 0; it < 200000; ++it) {
    const int rowgroups = (int)pick(1, 100000), chunks = (int)pick(1, 100000), cap = (int)pick(1, 8192);
    const int ks_cap = (int)pick(1, KS_MAX);
    int cps = 0;
    const int ks = choose_key_splits(rowgroups, chunks, cap, &cps, ks_cap);
    const sk_problem p{rowgroups, chunks, cap, ks_cap, 0, 0};
    expect(ks >= 1 && ks <= std::max(1, std::min(ks_cap, chunks / 2)) + 1 && cps >= 1, "split count in range", p);
    expect((long long)ks * cps >= chunks && (long long)(ks - 1) * cps < chunks, "splits cover every chunk once", p);
  }

  // eps
  const float es[] = {1e-3f, 1.f, 0.f, -1.f, INFINITY, NAN, 1e-45f};
  const bool ok[] = {true, true, false, false, false, false, false};
  for (int k = 0; k < 7; ++k) expect(eps_ok(es[k]) == ok[k], "eps validation", bad[0]);

  printf("host_check: %ld checks, %d failures\n", checks, failures);
  return failures ? 1 : 0;
}
