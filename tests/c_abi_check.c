/*
 * Plain-C user of the library's C ABI (include/sinkhorn.h), with no Python and
 * no torch: device memory from the HIP runtime, one sinkhorn_solve (fp32, eps
 * annealed) and one with bf16 inputs, checked against the fp64 oracle
 * (oracle/sinkhorn_oracle.c), then the host-side error paths.  Test
 * infrastructure: built by __graft_entry__.build(), run by
 * tests/test_gpu_c_abi.py.  Exit status 0 when every check passes.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "sinkhorn.h"

/* the oracle's solver (oracle/sinkhorn_oracle.c) */
void oracle_solve(int64_t n, int64_t m, int64_t d, const double* X, const double* Y, const double* a,
                  const double* b, const double* eps, int64_t n_eps, int64_t iters, double* f, double* g,
                  int nthreads);

#define HIP_OK(call)                                                                \
    do {                                                                            \
        hipError_t e_ = (call);                                                     \
        if (e_ != hipSuccess) {                                                     \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));      \
            exit(2);                                                                \
        }                                                                           \
    } while (0)

static int failures = 0;
static void expect(int ok, const char* what) {
    printf("%s: %s\n", ok ? "ok  " : "FAIL", what);
    if (!ok) ++failures;
}

/* test inputs: a 64-bit LCG, uniform in [-1, 1) */
static uint64_t state = 0x9E3779B97F4A7C15ull;
static double uniform(void) {
    state = state * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(state >> 11) * (1.0 / 9007199254740992.0) * 2.0 - 1.0;
}

/* bf16 bits of x by round to nearest even, and back */
static uint16_t to_bf16(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
static double from_bf16(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float x;
    memcpy(&x, &u, 4);
    return (double)x;
}

static void run_case(int64_t n, int64_t m, int64_t d, int bf16, const float* eps, int64_t n_eps, int64_t iters,
                     double bound_rel_eps, const char* name) {
    sk_problem p = {1, n, m, d, bf16 ? SK_BF16 : SK_FP32, SK_COST_SQEUCLID};
    size_t es = bf16 ? 2 : 4;
    void* hX = malloc((size_t)(n * d) * es);
    void* hY = malloc((size_t)(m * d) * es);
    double* X = malloc(sizeof(double) * (size_t)(n * d));
    double* Y = malloc(sizeof(double) * (size_t)(m * d));
    float* ha = malloc(sizeof(float) * (size_t)n);
    float* hb = malloc(sizeof(float) * (size_t)m);
    double* a = malloc(sizeof(double) * (size_t)n);
    double* b = malloc(sizeof(double) * (size_t)m);
    for (int64_t i = 0; i < n * d; ++i) {
        float v = (float)(uniform() / sqrt((double)d));
        if (bf16) {
            ((uint16_t*)hX)[i] = to_bf16(v);
            X[i] = from_bf16(((uint16_t*)hX)[i]);
        } else {
            ((float*)hX)[i] = v;
            X[i] = v;
        }
    }
    for (int64_t j = 0; j < m * d; ++j) {
        float v = (float)((uniform() + 0.3) / sqrt((double)d));
        if (bf16) {
            ((uint16_t*)hY)[j] = to_bf16(v);
            Y[j] = from_bf16(((uint16_t*)hY)[j]);
        } else {
            ((float*)hY)[j] = v;
            Y[j] = v;
        }
    }
    for (int64_t i = 0; i < n; ++i) ha[i] = (float)(1.0 / (double)n), a[i] = ha[i];
    for (int64_t j = 0; j < m; ++j) hb[j] = (float)(1.0 / (double)m), b[j] = hb[j];

    void *dX, *dY, *dws;
    float *da, *db, *df, *dg;
    size_t ws_bytes = sinkhorn_workspace_bytes(&p);
    expect(ws_bytes > 0, "workspace size of a valid problem");
    HIP_OK(hipMalloc(&dX, (size_t)(n * d) * es));
    HIP_OK(hipMalloc(&dY, (size_t)(m * d) * es));
    HIP_OK(hipMalloc((void**)&da, sizeof(float) * (size_t)n));
    HIP_OK(hipMalloc((void**)&db, sizeof(float) * (size_t)m));
    HIP_OK(hipMalloc((void**)&df, sizeof(float) * (size_t)n));
    HIP_OK(hipMalloc((void**)&dg, sizeof(float) * (size_t)m));
    HIP_OK(hipMalloc(&dws, ws_bytes));
    HIP_OK(hipMemcpy(dX, hX, (size_t)(n * d) * es, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dY, hY, (size_t)(m * d) * es, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(da, ha, sizeof(float) * (size_t)n, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(db, hb, sizeof(float) * (size_t)m, hipMemcpyHostToDevice));
    HIP_OK(hipMemset(df, 0, sizeof(float) * (size_t)n));
    HIP_OK(hipMemset(dg, 0, sizeof(float) * (size_t)m));
    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));

    sk_status st = sinkhorn_solve(&p, dX, dY, da, db, eps, n_eps, iters, df, dg, dws, ws_bytes, (void*)s);
    expect(st == SK_OK, "sinkhorn_solve returns SK_OK");
    if (st != SK_OK) printf("      %s\n", sinkhorn_last_error());
    HIP_OK(hipStreamSynchronize(s));
    float* f = malloc(sizeof(float) * (size_t)n);
    float* g = malloc(sizeof(float) * (size_t)m);
    HIP_OK(hipMemcpy(f, df, sizeof(float) * (size_t)n, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(g, dg, sizeof(float) * (size_t)m, hipMemcpyDeviceToHost));

    double* deps = malloc(sizeof(double) * (size_t)n_eps);
    for (int64_t k = 0; k < n_eps; ++k) deps[k] = eps[k];
    double* rf = calloc((size_t)n, sizeof(double));
    double* rg = calloc((size_t)m, sizeof(double));
    oracle_solve(n, m, d, X, Y, a, b, deps, n_eps, iters, rf, rg, 0);
    double ef = 0, eg = 0, mf = 0, mg = 0;
    for (int64_t i = 0; i < n; ++i) ef = fmax(ef, fabs(f[i] - rf[i])), mf = fmax(mf, fabs(rf[i]));
    for (int64_t j = 0; j < m; ++j) eg = fmax(eg, fabs(g[j] - rg[j])), mg = fmax(mg, fabs(rg[j]));
    double e_last = eps[n_eps - 1];
    double bf = bf16 ? bound_rel_eps * e_last : 1e-3 * e_last + 1e-5 * mf;
    double bg = bf16 ? bound_rel_eps * e_last : 1e-3 * e_last + 1e-5 * mg;
    char msg[256];
    snprintf(msg, sizeof msg, "%s: max|f - oracle| = %.3e (bound %.3e), max|g - oracle| = %.3e (bound %.3e)", name,
             ef, bf, eg, bg);
    expect(ef <= bf && eg <= bg, msg);

    /* host-side validation: nothing is launched, a status and a message come back */
    st = sinkhorn_solve(&p, dX, dY, da, db, eps, n_eps, iters, df, dg, dws, ws_bytes / 2, (void*)s);
    expect(st == SK_EWORKSPACE && strlen(sinkhorn_last_error()) > 0, "a small workspace is refused");
    float bad_eps = -1.f;
    st = sinkhorn_solve(&p, dX, dY, da, db, &bad_eps, 1, iters, df, dg, dws, ws_bytes, (void*)s);
    expect(st == SK_EINVAL, "a negative eps is refused");
    sk_problem q = p;
    q.d = 0;
    expect(sinkhorn_workspace_bytes(&q) == 0 && strlen(sinkhorn_last_error()) > 0, "d = 0 is refused");
    q.d = SK_MAX_D + 1;
    st = sinkhorn_solve(&q, dX, dY, da, db, eps, n_eps, iters, df, dg, dws, ws_bytes, (void*)s);
    expect(st != SK_OK, "d above SK_MAX_D is refused");

    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipStreamDestroy(s));
    hipFree(dX), hipFree(dY), hipFree(da), hipFree(db), hipFree(df), hipFree(dg), hipFree(dws);
    free(hX), free(hY), free(X), free(Y), free(ha), free(hb), free(a), free(b), free(f), free(g), free(deps);
    free(rf), free(rg);
}

int main(void) {
    int ndev = 0;
    HIP_OK(hipGetDeviceCount(&ndev));
    if (ndev < 1) {
        fprintf(stderr, "no GPU\n");
        return 2;
    }
    float sched[12];
    for (int k = 0; k < 12; ++k) sched[k] = (float)(0.5 * pow(0.1, k / 11.0));
    run_case(777, 513, 7, 0, sched, 12, 12, 0.0, "fp32, d = 7, eps annealed 0.5 -> 0.05");
    float e = 0.05f;
    run_case(600, 1030, 64, 1, &e, 1, 10, 2e-2, "bf16, d = 64, eps = 0.05");
    printf("%s (%d failures)\n", failures ? "C ABI check FAILED" : "C ABI check passed", failures);
    return failures ? 1 : 0;
}
