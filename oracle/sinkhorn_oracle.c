/*
 * Plain fp64 CPU oracle for log-domain Sinkhorn with squared-Euclidean cost.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously correct reference
 * that the GPU path is checked against.  Only the test-suite, the smoke check
 * and the benchmark's CPU-baseline leg may build or call it; the product path
 * never does.  It shares no code, header or table with the HIP library.
 *
 * What it computes (page "FlashSinkhorn: Trasporto Ottimo Entropico Consapevole delle I/O su GPU",
 * section "Metodologia", part "1. Riformulazione in Forma di Attenzione"): the
 * stabilised log-domain update
 *
 *     f_i <- -eps * LSE_j [ (g_j - C_ij)/eps + log b_j ],
 *     C_ij = ||x_i - y_j||^2          (squared Euclidean, no 1/2 factor),
 *
 * and, with the roles of the two clouds exchanged, the matching g update
 *
 *     g_j <- -eps * LSE_i [ (f_i - C_ij)/eps + log a_i ].
 *
 * The page states the f update and says the g update is its mirror image
 * (the bias gamma plays for g what delta plays for f); the mirror is written
 * here as the same routine called with the clouds swapped.  The cost is formed
 * explicitly from coordinate differences: no norm expansion, no dot products.
 * The log-sum-exp subtracts the exact maximum before exponentiating, which is
 * the definition of a stabilised LSE, not a streaming variant.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Number of threads the parallel loops below will use for a request of
 * `nthreads` (<= 0 means the OpenMP default). */
int oracle_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) return nthreads;
    return omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/* Squared Euclidean distance between two points of dimension d. */
static double sq_dist(const double* p, const double* q, int64_t d) {
    double c = 0.0;
    for (int64_t t = 0; t < d; ++t) {
        double diff = p[t] - q[t];
        c += diff * diff;
    }
    return c;
}

/*
 * One half-step of the log-domain Sinkhorn update (see the file header):
 *
 *   out[r] = -eps * LSE_j [ (h[j] - C(rows[r], j)) / eps + log w[j] ]
 *
 * P [np, d]: the points that own the potential being computed (rows),
 * Q [nq, d]: the other cloud, w [nq] its weights, h [nq] its potential.
 * rows: optional list of `nsel` row indices into P (NULL = all np rows, nsel = np).
 * A zero weight contributes log 0 = -inf, i.e. removes that point; if every
 * term is removed the result is +inf.
 */
void oracle_half_step(int64_t np_, int64_t nq, int64_t d, const double* P, const double* Q,
                      const double* w, const double* h, double eps,
                      const int64_t* rows, int64_t nsel, double* out, int nthreads) {
    if (rows == NULL) nsel = np_;
    double* logw = (double*)malloc(sizeof(double) * (size_t)(nq > 0 ? nq : 1));
    for (int64_t j = 0; j < nq; ++j) logw[j] = log(w[j]);
    int nt = oracle_threads(nthreads);

#ifdef _OPENMP
#pragma omp parallel num_threads(nt)
#endif
    {
        double* v = (double*)malloc(sizeof(double) * (size_t)(nq > 0 ? nq : 1));
#ifdef _OPENMP
#pragma omp for schedule(static)
#endif
        for (int64_t r = 0; r < nsel; ++r) {
            int64_t i = rows ? rows[r] : r;
            const double* p = P + i * d;
            double vmax = -INFINITY;
            for (int64_t j = 0; j < nq; ++j) {
                double c = sq_dist(p, Q + j * d, d);
                v[j] = (h[j] - c) / eps + logw[j];
                if (v[j] > vmax) vmax = v[j];
            }
            if (vmax == -INFINITY) {
                out[r] = INFINITY;
                continue;
            }
            double s = 0.0;
            for (int64_t j = 0; j < nq; ++j) s += exp(v[j] - vmax);
            out[r] = -eps * (vmax + log(s));
        }
        free(v);
    }
    (void)nt;
    free(logw);
}

/*
 * Sinkhorn iterations, alternating: f from g, then g from the new f
 * (page "FlashSinkhorn: Trasporto Ottimo Entropico Consapevole delle I/O su GPU", section
 * "Metodologia", part "1. Riformulazione in Forma di Attenzione";
 * the solver repeats the two updates a fixed number of times).
 * X [n, d], Y [m, d], a [n], b [m]; f [n], g [m] are in/out: only the
 * incoming g matters because every iteration starts with the f update.
 * eps: n_eps values; n_eps == 1 means constant, otherwise iteration k uses eps[k]
 * for both of its half-steps.
 */
void oracle_solve(int64_t n, int64_t m, int64_t d, const double* X, const double* Y,
                  const double* a, const double* b, const double* eps, int64_t n_eps,
                  int64_t iters, double* f, double* g, int nthreads) {
    for (int64_t k = 0; k < iters; ++k) {
        double e = (n_eps == 1) ? eps[0] : eps[k];
        oracle_half_step(n, m, d, X, Y, b, g, e, NULL, n, f, nthreads);
        oracle_half_step(m, n, d, Y, X, a, f, e, NULL, m, g, nthreads);
    }
}

/*
 * Marginals of the transport plan P_ij = a_i b_j exp((f_i + g_j - C_ij)/eps),
 * formed element by element: row[i] = sum_j P_ij, col[j] = sum_i P_ij.
 */
void oracle_plan_marginals(int64_t n, int64_t m, int64_t d, const double* X, const double* Y,
                           const double* a, const double* b, const double* f, const double* g,
                           double eps, double* row, double* col, int nthreads) {
    int nt = oracle_threads(nthreads);
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(nt)
#endif
    for (int64_t i = 0; i < n; ++i) {
        double s = 0.0;
        for (int64_t j = 0; j < m; ++j) {
            double c = sq_dist(X + i * d, Y + j * d, d);
            s += a[i] * b[j] * exp((f[i] + g[j] - c) / eps);
        }
        row[i] = s;
    }
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(nt)
#endif
    for (int64_t j = 0; j < m; ++j) {
        double s = 0.0;
        for (int64_t i = 0; i < n; ++i) {
            double c = sq_dist(X + i * d, Y + j * d, d);
            s += a[i] * b[j] * exp((f[i] + g[j] - c) / eps);
        }
        col[j] = s;
    }
    (void)nt;
}

/*
 * Transport application for the rows of P (page "FlashSinkhorn: Trasporto Ottimo Entropico
 * Consapevole delle I/O su GPU", section "Metodologia", part "3. Differenziazione e Ottimizzazione
 * del Secondo Ordine": the barycentric projection and the gradient are weighted
 * averages over the transport plan, evaluated without forming the plan).
 *
 * With the plan entries pi_rj = wp_r wq_j exp((hp_r + hq_j - C_rj)/eps):
 *   mass[r]        = sum_j pi_rj
 *   bary[r*d + t]  = sum_j pi_rj Q_jt / mass[r]       (barycentric projection of P_r)
 *   grad[r*d + t]  = sum_j pi_rj * 2 (P_rt - Q_jt)    (derivative of sum_j pi_rj C_rj in P_rt,
 *                                                      the plan held fixed)
 * The row's largest exponent is factored out of every pi_rj (exact in exact
 * arithmetic); each output is then the plain sum over j written above.
 * rows: optional list of nsel row indices (NULL = all np rows).  grad and mass
 * may be NULL.
 */
void oracle_transport(int64_t np_, int64_t nq, int64_t d, const double* P, const double* Q,
                      const double* wp, const double* wq, const double* hp, const double* hq,
                      double eps, const int64_t* rows, int64_t nsel, double* bary, double* grad,
                      double* mass, int nthreads) {
    if (rows == NULL) nsel = np_;
    int nt = oracle_threads(nthreads);
#ifdef _OPENMP
#pragma omp parallel num_threads(nt)
#endif
    {
        double* v = (double*)malloc(sizeof(double) * (size_t)(nq > 0 ? nq : 1));
#ifdef _OPENMP
#pragma omp for schedule(static)
#endif
        for (int64_t r = 0; r < nsel; ++r) {
            int64_t i = rows ? rows[r] : r;
            const double* p = P + i * d;
            /* log pi_ij = log wp_i + hp_i/eps + v_j with v_j = (hq_j - C_ij)/eps + log wq_j */
            double vmax = -INFINITY;
            for (int64_t j = 0; j < nq; ++j) {
                v[j] = (hq[j] - sq_dist(p, Q + j * d, d)) / eps + log(wq[j]);
                if (v[j] > vmax) vmax = v[j];
            }
            double lead = log(wp[i]) + hp[i] / eps + vmax; /* pi_ij = exp(lead) * exp(v_j - vmax) */
            double s = 0.0;
            for (int64_t j = 0; j < nq; ++j) s += exp(v[j] - vmax);
            for (int64_t t = 0; t < d; ++t) {
                double num = 0.0, gr = 0.0;
                for (int64_t j = 0; j < nq; ++j) {
                    double pij = exp(lead + v[j] - vmax);
                    num += exp(v[j] - vmax) * Q[j * d + t];
                    gr += pij * 2.0 * (p[t] - Q[j * d + t]);
                }
                bary[r * d + t] = num / s;
                if (grad) grad[r * d + t] = gr;
            }
            if (mass) mass[r] = exp(lead) * s;
        }
        free(v);
    }
    (void)nt;
}

/*
 * Plan applied to a matrix (page "FlashSinkhorn: Trasporto Ottimo Entropico Consapevole delle I/O su GPU",
 * section "Metodologia", part "3. Differenziazione e Ottimizzazione del Secondo Ordine": vector- and
 * matrix-transport products):
 *   out[r*c + k] = sum_j pi_rj V[j*c + k],  pi_rj = wp_r wq_j exp((hp_r + hq_j - C_rj)/eps)
 * for the selected rows r of P (rows NULL = all).  V is [nq, c].
 */
void oracle_apply_plan(int64_t np_, int64_t nq, int64_t d, const double* P, const double* Q,
                       const double* wp, const double* wq, const double* hp, const double* hq,
                       double eps, const double* V, int64_t c, const int64_t* rows, int64_t nsel,
                       double* out, int nthreads) {
    if (rows == NULL) nsel = np_;
    int nt = oracle_threads(nthreads);
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(nt)
#endif
    for (int64_t r = 0; r < nsel; ++r) {
        int64_t i = rows ? rows[r] : r;
        const double* p = P + i * d;
        for (int64_t k = 0; k < c; ++k) out[r * c + k] = 0.0;
        for (int64_t j = 0; j < nq; ++j) {
            double pij = wp[i] * wq[j] * exp((hp[i] + hq[j] - sq_dist(p, Q + j * d, d)) / eps);
            for (int64_t k = 0; k < c; ++k) out[r * c + k] += pij * V[j * c + k];
        }
    }
    (void)nt;
}
