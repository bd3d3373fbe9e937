"""Pins for the oracle's transport application (barycentric projection, gradient, row mass).

Page "FlashSinkhorn: Trasporto Ottimo Entropico Consapevole delle I/O su GPU", section
"Metodologia", part "3. Differenziazione e Ottimizzazione del Secondo Ordine": the barycentric
projection and the gradient are
weighted averages over the transport plan.  The pages print no numbers for
them, so each pin comes from mathematics the definitions fix:

* m = 1: every row is sent to the single target (closed form),
* eps -> infinity with zero potentials: the plan factorises, the projection is
  the b-weighted mean of Y,
* eps -> 0 at converged potentials: the projection is the optimal assignment's
  partner (brute force over permutations),
* the gradient equals finite differences of the converged dual value
  <a,f> + <b,g> in each coordinate of X (envelope theorem),
* translating both clouds together leaves the cost unchanged, so the X and Y
  gradients of any plan sum to zero,
* a dense numpy brute force of the plan on tiny inputs.
"""

import itertools

import numpy as np
import pytest

import oracle
from log_domain_sinkhorn_half_amd.inputs import make_case, random_potential


def _dense(X, Y, a, b, f, g, eps):
    C = ((X[:, None, :] - Y[None, :, :]) ** 2).sum(-1)
    return a[:, None] * b[None, :] * np.exp((f[:, None] + g[None, :] - C) / eps)


def test_single_target_closed_form():
    p = make_case(9, 1, 3, eps=0.2, seed=11)
    X, Y, a, b = p.X[0].astype(np.float64), p.Y[0].astype(np.float64), p.a[0], p.b[0]
    f = random_potential(9, 1, scale=0.3).astype(np.float64)
    g = np.array([0.7])
    bary, grad, mass = oracle.transport_x(X, Y, a, b, f, g, 0.2)
    c = ((X - Y[0]) ** 2).sum(1)
    m_ref = a * b[0] * np.exp((f + g[0] - c) / 0.2)
    np.testing.assert_allclose(bary, np.broadcast_to(Y[0], X.shape), rtol=0, atol=1e-15)
    np.testing.assert_allclose(mass, m_ref, rtol=1e-13)
    np.testing.assert_allclose(grad, 2 * m_ref[:, None] * (X - Y[0]), rtol=1e-12, atol=1e-300)


def test_large_eps_weighted_mean():
    p = make_case(6, 40, 2, eps=1.0, weights="softmax", seed=12)
    X, Y, a, b = p.X[0].astype(np.float64), p.Y[0].astype(np.float64), p.a[0].astype(np.float64), p.b[0].astype(np.float64)
    eps = 1e9
    bary, _, mass = oracle.transport_x(X, Y, a, b, np.zeros(6), np.zeros(40), eps)
    mean = (b[:, None] * Y).sum(0) / b.sum()
    # first-order correction is O(C/eps) relative
    np.testing.assert_allclose(bary, np.broadcast_to(mean, bary.shape), rtol=0, atol=1e-7)
    np.testing.assert_allclose(mass, a * b.sum(), rtol=1e-7)


def test_small_eps_assignment_partner():
    rng = np.random.default_rng(13)
    n = 6
    X = rng.random((n, 2))
    perm = rng.permutation(n)
    Y = X[perm] + 0.3 * rng.standard_normal((n, 2))
    a = np.full(n, 1.0 / n)
    b = np.full(n, 1.0 / n)
    C = ((X[:, None, :] - Y[None, :, :]) ** 2).sum(-1)
    best = min(itertools.permutations(range(n)), key=lambda s: sum(C[i, s[i]] for i in range(n)))
    costs = sorted(sum(C[i, s[i]] for i in range(n)) for s in itertools.permutations(range(n)))
    assert costs[1] - costs[0] > 1e-2  # a unique optimum with a clear gap
    eps = 5e-4
    f, g = oracle.solve(X, Y, a, b, eps, 20000)
    bary, _, mass = oracle.transport_x(X, Y, a, b, f, g, eps)
    # the blur of the entropic plan and the unconverged rows are both O(eps) here
    np.testing.assert_allclose(mass, a, rtol=2e-4)
    np.testing.assert_allclose(bary, Y[list(best)], atol=2e-4)
    bary_y, _, mass_y = oracle.transport_y(X, Y, a, b, f, g, eps)
    np.testing.assert_allclose(mass_y, b, rtol=1e-12)  # columns: exact after the last g update
    inv = np.argsort(best)
    np.testing.assert_allclose(bary_y, X[inv], atol=2e-4)


@pytest.mark.parametrize("side", ["x", "y"])
def test_gradient_is_derivative_of_converged_dual(side):
    rng = np.random.default_rng(14)
    n, m, d, eps = 5, 4, 2, 0.5
    X = rng.random((n, d))
    Y = rng.random((m, d)) + 0.2
    a = np.array([0.1, 0.3, 0.2, 0.25, 0.15])
    b = np.array([0.4, 0.1, 0.3, 0.2])

    def value(X_, Y_):
        f, g = oracle.solve(X_, Y_, a, b, eps, 400)
        return a @ f + b @ g

    f, g = oracle.solve(X, Y, a, b, eps, 400)
    if side == "x":
        _, grad, _ = oracle.transport_x(X, Y, a, b, f, g, eps)
        base = X
    else:
        _, grad, _ = oracle.transport_y(X, Y, a, b, f, g, eps)
        base = Y
    h = 1e-5
    fd = np.zeros_like(base)
    for i in range(base.shape[0]):
        for t in range(d):
            up, dn = base.copy(), base.copy()
            up[i, t] += h
            dn[i, t] -= h
            if side == "x":
                fd[i, t] = (value(up, Y) - value(dn, Y)) / (2 * h)
            else:
                fd[i, t] = (value(X, up) - value(X, dn)) / (2 * h)
    np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-8)


def test_translation_balance_of_gradients():
    p = make_case(12, 17, 3, eps=0.3, weights="softmax", seed=15)
    X, Y, a, b = (v[0].astype(np.float64) for v in (p.X, p.Y, p.a, p.b))
    f = random_potential(12, 2, scale=0.5).astype(np.float64)
    g = random_potential(17, 3, scale=0.5).astype(np.float64)
    _, gx, _ = oracle.transport_x(X, Y, a, b, f, g, 0.3)
    _, gy, _ = oracle.transport_y(X, Y, a, b, f, g, 0.3)
    scale = np.abs(gx).sum() + np.abs(gy).sum()
    np.testing.assert_allclose(gx.sum(0) + gy.sum(0), 0.0, atol=1e-13 * scale)


@pytest.mark.parametrize("eps", [0.05, 1.0])
def test_dense_brute_force(eps):
    p = make_case(8, 10, 3, eps=eps, weights="softmax", seed=16)
    X, Y, a, b = (v[0].astype(np.float64) for v in (p.X, p.Y, p.a, p.b))
    f = random_potential(8, 4, scale=0.1).astype(np.float64)
    g = random_potential(10, 5, scale=0.1).astype(np.float64)
    P = _dense(X, Y, a, b, f, g, eps)
    bary, grad, mass = oracle.transport_x(X, Y, a, b, f, g, eps)
    np.testing.assert_allclose(mass, P.sum(1), rtol=1e-12)
    np.testing.assert_allclose(bary, (P @ Y) / P.sum(1)[:, None], rtol=1e-12)
    np.testing.assert_allclose(grad, 2 * (P.sum(1)[:, None] * X - P @ Y), rtol=1e-10, atol=1e-14)
    bary_y, grad_y, mass_y = oracle.transport_y(X, Y, a, b, f, g, eps)
    np.testing.assert_allclose(mass_y, P.sum(0), rtol=1e-12)
    np.testing.assert_allclose(bary_y, (P.T @ X) / P.sum(0)[:, None], rtol=1e-12)
    np.testing.assert_allclose(grad_y, 2 * (P.sum(0)[:, None] * Y - P.T @ X), rtol=1e-10, atol=1e-14)


def test_row_subset_matches_full():
    p = make_case(20, 9, 2, eps=0.1, seed=17)
    X, Y, a, b = (v[0].astype(np.float64) for v in (p.X, p.Y, p.a, p.b))
    f = random_potential(20, 6, scale=0.2).astype(np.float64)
    g = random_potential(9, 7, scale=0.2).astype(np.float64)
    full = oracle.transport_x(X, Y, a, b, f, g, 0.1)
    rows = np.array([19, 0, 7])
    sub = oracle.transport_x(X, Y, a, b, f, g, 0.1, rows=rows)
    for u, v in zip(full, sub):
        np.testing.assert_array_equal(u[rows], v)
