"""Pins for the fp64 CPU oracle, each against something other than the oracle.

The pages print no worked example, so every pin here comes from mathematics the
method fixes (page "FlashSinkhorn: Trasporto Ottimo Entropico Consapevole delle I/O su GPU", section
"Metodologia", part "1. Riformulazione in Forma di Attenzione": the stabilised log-domain update
with squared-Euclidean cost):

* plan marginals formed by brute force in numpy after each half-step,
* closed forms for m = 1 and n = 1 (the latter through scipy's logsumexp),
* the hard c-transform limit of a half-step as eps -> 0,
* the second-order cumulant expansion of a half-step as eps -> infinity,
* gauge invariance (f + c, g - c), monotone dual ascent, the eps -> 0
  assignment limit against brute force over permutations,
* invariance of the cost under translation / rotation, permutation equivariance.
"""

import itertools

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle
from log_domain_sinkhorn_half_amd.inputs import make_case, random_potential


def _cost(X, Y):
    X = np.asarray(X, np.float64)
    Y = np.asarray(Y, np.float64)
    return ((X[:, None, :] - Y[None, :, :]) ** 2).sum(-1)


def _plan(X, Y, a, b, f, g, eps):
    C = _cost(X, Y)
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return a[:, None] * b[None, :] * np.exp((f[:, None] + g[None, :] - C) / eps)


def _dual(X, Y, a, b, f, g, eps):
    C = _cost(X, Y)
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    K = a[:, None] * b[None, :] * (np.exp((f[:, None] + g[None, :] - C) / eps) - 1.0)
    return a @ f + b @ g - eps * K.sum()


CASES = [
    dict(n=7, m=11, d=3, eps=0.05, weights="softmax", seed=1),
    dict(n=13, m=5, d=4, eps=1.0, weights="uniform", seed=2),
    dict(n=16, m=16, d=2, eps=0.3, weights="softmax", seed=3),
    dict(n=9, m=14, d=1, eps=7.0, weights="softmax", seed=4),
]


@pytest.mark.parametrize("cfg", CASES)
def test_f_step_rows_sum_to_a(cfg):
    p = make_case(cfg["n"], cfg["m"], cfg["d"], eps=cfg["eps"], weights=cfg["weights"],
                  seed=cfg["seed"])
    X, Y, a, b = p.X[0], p.Y[0], p.a[0], p.b[0]
    g = random_potential(p.m, cfg["seed"], scale=0.7).astype(np.float64)
    f = oracle.half_step_f(X, Y, b, g, cfg["eps"])
    P = _plan(X, Y, a, b, f, g, cfg["eps"])
    np.testing.assert_allclose(P.sum(1), a.astype(np.float64), rtol=1e-11, atol=0)


@pytest.mark.parametrize("cfg", CASES)
def test_g_step_columns_sum_to_b(cfg):
    p = make_case(cfg["n"], cfg["m"], cfg["d"], eps=cfg["eps"], weights=cfg["weights"],
                  seed=cfg["seed"])
    X, Y, a, b = p.X[0], p.Y[0], p.a[0], p.b[0]
    f = random_potential(p.n, cfg["seed"] + 50, scale=0.7).astype(np.float64)
    g = oracle.half_step_g(X, Y, a, f, cfg["eps"])
    P = _plan(X, Y, a, b, f, g, cfg["eps"])
    np.testing.assert_allclose(P.sum(0), b.astype(np.float64), rtol=1e-11, atol=0)


def test_m1_closed_form_pins_the_cost_convention():
    # One target point with weight 1: from g = 0 the f update is exactly the
    # squared distance (no 1/2), and the g update is -eps*log(sum a) = 0.
    rng = np.random.default_rng(7)
    X = rng.standard_normal((9, 3))
    Y = rng.standard_normal((1, 3))
    a = np.full(9, 1.0 / 9)
    b = np.ones(1)
    for eps in (0.01, 0.5, 3.0):
        f, g = oracle.solve(X, Y, a, b, eps, iters=1)
        C = ((X - Y[0]) ** 2).sum(1)
        np.testing.assert_allclose(f, C, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(g, [0.0], atol=1e-13)
        f5, g5 = oracle.solve(X, Y, a, b, eps, iters=5)
        np.testing.assert_allclose(f5, C, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(g5, [0.0], atol=1e-13)


def test_n1_closed_form_softmin():
    rng = np.random.default_rng(8)
    X = rng.standard_normal((1, 4))
    Y = rng.standard_normal((12, 4))
    a = np.ones(1)
    b = rng.random(12)
    b /= b.sum()
    C = ((Y - X[0]) ** 2).sum(1)
    for eps in (0.05, 0.4, 2.0):
        f, g = oracle.solve(X, Y, a, b, eps, iters=1)
        f_ref = -eps * logsumexp(-C / eps, b=b)
        np.testing.assert_allclose(f, [f_ref], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(g, C - f_ref, rtol=1e-12, atol=1e-12)
        # fixed after the first iteration
        f3, g3 = oracle.solve(X, Y, a, b, eps, iters=3)
        np.testing.assert_allclose(f3, f, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(g3, g, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("eps", [2e-3, 1e-2])
def test_small_eps_hard_c_transform(eps):
    # f_i = -eps*LSE_j[v_ij], v_ij = (g_j - C_ij)/eps + log b_j; with M_i = eps*max_j v_ij,
    # max <= LSE <= max + log m gives -M_i - eps*log(m) <= f_i <= -M_i.
    p = make_case(10, 15, 3, weights="softmax", seed=11)
    X, Y, b = p.X[0], p.Y[0], p.b[0].astype(np.float64)
    g = random_potential(15, 11, scale=0.5).astype(np.float64)
    f = oracle.half_step_f(X, Y, b, g, eps)
    C = _cost(X, Y)
    M = (g[None, :] - C + eps * np.log(b)[None, :]).max(1)
    assert np.all(f <= -M + 1e-12)
    assert np.all(f >= -M - eps * np.log(15) - 1e-12)


def test_large_eps_cumulant_expansion():
    # -eps*log E_b[exp(-C/eps)] = E_b[C] - Var_b[C]/(2 eps) + O(eps^-2) (from g = 0)
    p = make_case(6, 20, 3, weights="softmax", seed=12)
    X, Y, b = p.X[0], p.Y[0], p.b[0].astype(np.float64)
    b = b / b.sum()
    C = _cost(X, Y)
    mean = C @ b
    var = ((C - mean[:, None]) ** 2) @ b
    third = np.abs((C - mean[:, None]) ** 3) @ b
    for eps in (50.0, 500.0):
        f = oracle.half_step_f(X, Y, b, np.zeros(20), eps)
        assert np.all(f <= mean + 1e-12)  # Jensen
        err = np.abs(f - (mean - var / (2 * eps)))
        assert np.all(err <= third / eps ** 2 + 1e-12), (err, third / eps ** 2)


def test_gauge_shift_invariance():
    p = make_case(12, 9, 3, eps=0.2, weights="softmax", seed=13)
    X, Y, a, b = p.X[0], p.Y[0], p.a[0], p.b[0]
    c = 0.37
    f0, g0 = oracle.solve(X, Y, a, b, 0.2, iters=6)
    f1, g1 = oracle.solve(X, Y, a, b, 0.2, iters=6, g0=np.full(9, -c))
    np.testing.assert_allclose(f1, f0 + c, rtol=0, atol=1e-12)
    np.testing.assert_allclose(g1, g0 - c, rtol=0, atol=1e-12)
    d0 = a.astype(np.float64) @ f0 + b.astype(np.float64) @ g0
    d1 = a.astype(np.float64) @ f1 + b.astype(np.float64) @ g1
    # sum(a) and sum(b) are 1 up to float32 rounding of the stored weights
    assert abs(d1 - d0) <= c * (abs(a.astype(np.float64).sum() - b.astype(np.float64).sum())) + 1e-12


def test_dual_ascent_and_unit_mass():
    p = make_case(14, 10, 2, eps=0.1, weights="softmax", seed=14)
    X, Y, a, b = p.X[0], p.Y[0], p.a[0], p.b[0]
    eps = 0.1
    g = np.zeros(10)
    f = np.zeros(14)
    prev = _dual(X, Y, a, b, f, g, eps)
    for _ in range(15):
        f = oracle.half_step_f(X, Y, b, g, eps)
        cur = _dual(X, Y, a, b, f, g, eps)
        assert cur >= prev - 1e-12
        assert abs(_plan(X, Y, a, b, f, g, eps).sum() - a.astype(np.float64).sum()) < 1e-12
        prev = cur
        g = oracle.half_step_g(X, Y, a, f, eps)
        cur = _dual(X, Y, a, b, f, g, eps)
        assert cur >= prev - 1e-12
        assert abs(_plan(X, Y, a, b, f, g, eps).sum() - b.astype(np.float64).sum()) < 1e-12
        prev = cur


@pytest.mark.parametrize("seed", [21, 22, 23])
def test_small_eps_matches_assignment(seed):
    n = 5
    rng = np.random.default_rng(seed)
    X = rng.random((n, 2))
    Y = rng.random((n, 2))
    a = np.full(n, 1.0 / n)
    b = np.full(n, 1.0 / n)
    C = _cost(X, Y)
    ot0 = min(sum(C[i, s[i]] for i in range(n)) for s in itertools.permutations(range(n))) / n
    eps = 0.01
    f, g = oracle.solve(X, Y, a, b, eps, iters=20000)
    ra, cb = oracle.marginal_error(X, Y, a, b, f, g, eps)
    assert ra < 1e-5 and cb < 1e-12  # slow near-degenerate cases converge to ~1e-6
    D = a @ f + b @ g
    assert ot0 - 1e-6 <= D <= ot0 + eps * np.log(n) + 1e-12, (D, ot0)


def test_cost_invariances_and_permutation():
    p = make_case(11, 8, 3, eps=0.15, weights="softmax", seed=15)
    X, Y, a, b = (v[0].astype(np.float64) for v in (p.X, p.Y, p.a, p.b))
    f, g = oracle.solve(X, Y, a, b, 0.15, iters=7)
    t = np.array([0.3, -1.1, 2.0])
    ft, gt = oracle.solve(X + t, Y + t, a, b, 0.15, iters=7)
    np.testing.assert_allclose(ft, f, atol=1e-11)
    np.testing.assert_allclose(gt, g, atol=1e-11)
    Q, _ = np.linalg.qr(np.random.default_rng(3).standard_normal((3, 3)))
    fr, gr = oracle.solve(X @ Q.T, Y @ Q.T, a, b, 0.15, iters=7)
    np.testing.assert_allclose(fr, f, atol=1e-11)
    np.testing.assert_allclose(gr, g, atol=1e-11)
    perm = np.random.default_rng(4).permutation(11)
    fp, gp = oracle.solve(X[perm], Y, a[perm], b, 0.15, iters=7)
    np.testing.assert_allclose(fp, f[perm], atol=1e-11)
    np.testing.assert_allclose(gp, g, atol=1e-11)


def test_marginals_match_dense_plan():
    p = make_case(9, 12, 3, eps=0.3, weights="softmax", seed=16)
    X, Y, a, b = p.X[0], p.Y[0], p.a[0], p.b[0]
    f = random_potential(9, 1).astype(np.float64)
    g = random_potential(12, 2).astype(np.float64)
    row, col = oracle.plan_marginals(X, Y, a, b, f, g, 0.3)
    P = _plan(X, Y, a, b, f, g, 0.3)
    np.testing.assert_allclose(row, P.sum(1), rtol=1e-13)
    np.testing.assert_allclose(col, P.sum(0), rtol=1e-13)


def test_row_subset_and_batch_agree_with_full():
    p = make_case(40, 30, 4, batch=3, eps=0.2, weights="softmax", seed=17)
    f, g = oracle.solve(p.X, p.Y, p.a, p.b, 0.2, iters=3)
    for k in range(3):
        fk, gk = oracle.solve(p.X[k], p.Y[k], p.a[k], p.b[k], 0.2, iters=3)
        np.testing.assert_array_equal(f[k], fk)
        np.testing.assert_array_equal(g[k], gk)
    rows = np.array([0, 39, 7, 7, 21])
    gin = random_potential(30, 5).astype(np.float64)
    full = oracle.half_step_f(p.X[0], p.Y[0], p.b[0], gin, 0.2)
    sub = oracle.half_step_f(p.X[0], p.Y[0], p.b[0], gin, 0.2, rows=rows)
    np.testing.assert_array_equal(sub, full[rows])


def test_zero_weight_removes_point():
    p = make_case(6, 7, 2, eps=0.2, weights="softmax", seed=18)
    X, Y, a = p.X[0], p.Y[0], p.a[0].astype(np.float64)
    b = p.b[0].astype(np.float64).copy()
    b[3] = 0.0
    g = random_potential(7, 6).astype(np.float64)
    f = oracle.half_step_f(X, Y, b, g, 0.2)
    keep = [0, 1, 2, 4, 5, 6]
    f2 = oracle.half_step_f(X, Y[keep], b[keep], g[keep], 0.2)
    np.testing.assert_allclose(f, f2, rtol=1e-14, atol=1e-14)


def test_annealed_schedule_uses_per_iteration_eps():
    p = make_case(8, 6, 3, weights="softmax", seed=19)
    X, Y, a, b = p.X[0], p.Y[0], p.a[0], p.b[0]
    sched = np.array([1.0, 0.5, 0.2])
    f, g = oracle.solve(X, Y, a, b, sched, iters=3)
    f2 = np.zeros(8)
    g2 = np.zeros(6)
    for e in sched:
        f2 = oracle.half_step_f(X, Y, b, g2, e)
        g2 = oracle.half_step_g(X, Y, a, f2, e)
    np.testing.assert_array_equal(f, f2)
    np.testing.assert_array_equal(g, g2)
