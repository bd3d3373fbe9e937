"""Pins for the oracle's cosine cost (page "FlashSinkhorn: Trasporto Ottimo Entropico Consapevole
delle I/O su GPU", section "Significato e Affermazioni": cosine distance after normalisation).

The oracle runs the squared-Euclidean routines on normalised clouds, so the pins
check the normalisation and the chain rule against independent facts:

* d = 2: the cost between unit vectors at angles t_i, s_j is 2 - 2 cos(t_i - s_j)
  (closed form through trigonometry, no dot products),
* positive rescaling of any point leaves the potentials unchanged,
* the gradient in the raw points equals finite differences of the converged dual
  value, and is orthogonal to its point (the cost ignores radial motion).
"""

import numpy as np
from scipy.special import logsumexp

import oracle


def test_two_d_closed_form_cost():
    rng = np.random.default_rng(21)
    t = rng.uniform(0, 2 * np.pi, 9)
    s = rng.uniform(0, 2 * np.pi, 7)
    rx = rng.uniform(0.1, 5.0, 9)
    ry = rng.uniform(0.1, 5.0, 7)
    X = np.stack([rx * np.cos(t), rx * np.sin(t)], 1)
    Y = np.stack([ry * np.cos(s), ry * np.sin(s)], 1)
    b = rng.dirichlet(np.ones(7))
    g = rng.standard_normal(7) * 0.3
    eps = 0.2
    f = oracle.half_step_f(oracle.normalize(X), oracle.normalize(Y), b, g, eps)
    C = 2.0 - 2.0 * np.cos(t[:, None] - s[None, :])
    ref = -eps * logsumexp((g[None, :] - C) / eps + np.log(b)[None, :], axis=1)
    np.testing.assert_allclose(f, ref, rtol=0, atol=1e-13)


def test_rescaling_points_leaves_potentials_unchanged():
    rng = np.random.default_rng(22)
    X = rng.standard_normal((12, 5))
    Y = rng.standard_normal((10, 5)) + 0.3
    a = rng.dirichlet(np.ones(12))
    b = rng.dirichlet(np.ones(10))
    f1, g1 = oracle.solve(oracle.normalize(X), oracle.normalize(Y), a, b, 0.1, 30)
    X2 = X * rng.uniform(0.01, 100.0, (12, 1))
    Y2 = Y * rng.uniform(0.01, 100.0, (10, 1))
    f2, g2 = oracle.solve(oracle.normalize(X2), oracle.normalize(Y2), a, b, 0.1, 30)
    np.testing.assert_allclose(f1, f2, atol=1e-12)
    np.testing.assert_allclose(g1, g2, atol=1e-12)


def test_zero_point_normalises_to_zero():
    X = np.array([[0.0, 0.0, 0.0], [3.0, 4.0, 0.0]])
    Xh = oracle.normalize(X)
    np.testing.assert_array_equal(Xh[0], 0.0)
    np.testing.assert_allclose(Xh[1], [0.6, 0.8, 0.0], rtol=1e-15)


def test_raw_gradient_matches_finite_differences_and_is_tangent():
    rng = np.random.default_rng(23)
    n, m, d, eps = 5, 4, 3, 0.4
    X = rng.standard_normal((n, d))
    Y = rng.standard_normal((m, d))
    a = rng.dirichlet(np.ones(n))
    b = rng.dirichlet(np.ones(m))

    def value(X_):
        f, g = oracle.solve(oracle.normalize(X_), oracle.normalize(Y), a, b, eps, 600)
        return a @ f + b @ g

    Xh, Yh = oracle.normalize(X), oracle.normalize(Y)
    f, g = oracle.solve(Xh, Yh, a, b, eps, 600)
    _, grad_hat, _ = oracle.transport_x(Xh, Yh, a, b, f, g, eps)
    grad = oracle.cosine_grad(X, grad_hat)
    h = 1e-6
    fd = np.zeros_like(X)
    for i in range(n):
        for t in range(d):
            up, dn = X.copy(), X.copy()
            up[i, t] += h
            dn[i, t] -= h
            fd[i, t] = (value(up) - value(dn)) / (2 * h)
    np.testing.assert_allclose(grad, fd, rtol=1e-5, atol=1e-8)
    np.testing.assert_allclose((grad * X).sum(1), 0.0, atol=1e-12)
