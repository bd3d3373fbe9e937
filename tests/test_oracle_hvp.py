"""Pins for the oracle's plan application and Hessian-vector product (page
"FlashSinkhorn: Trasporto Ottimo Entropico Consapevole delle I/O su GPU", section "Metodologia",
part "3. Differenziazione e Ottimizzazione del Secondo Ordine": vector- and matrix-transport
products, streaming HVP).

* apply_plan: a dense numpy plan; applied to the other cloud it equals
  mass * barycentric projection from the transport routine;
* hvp_x: central finite differences of the converged gradient along the
  direction; symmetry <U, H V> = <V, H U>; m = 1 closed form H V = 2 a v (the plan
  cannot move); eps -> infinity limit 2 a_i (sum b) v_i.
"""

import numpy as np
import pytest

import oracle
from log_domain_sinkhorn_half_amd.inputs import make_case, random_potential


def _dense(X, Y, a, b, f, g, eps):
    C = ((X[:, None, :] - Y[None, :, :]) ** 2).sum(-1)
    return a[:, None] * b[None, :] * np.exp((f[:, None] + g[None, :] - C) / eps)


def test_apply_plan_dense_and_consistent_with_transport():
    p = make_case(9, 11, 3, eps=0.3, weights="softmax", seed=31)
    X, Y, a, b = (v[0].astype(np.float64) for v in (p.X, p.Y, p.a, p.b))
    f = random_potential(9, 8, scale=0.2).astype(np.float64)
    g = random_potential(11, 9, scale=0.2).astype(np.float64)
    V = np.random.default_rng(1).standard_normal((11, 4))
    U = np.random.default_rng(2).standard_normal(9)
    P = _dense(X, Y, a, b, f, g, 0.3)
    np.testing.assert_allclose(oracle.apply_plan_x(X, Y, a, b, f, g, 0.3, V), P @ V, rtol=1e-12)
    np.testing.assert_allclose(oracle.apply_plan_y(X, Y, a, b, f, g, 0.3, U), P.T @ U, rtol=1e-12)
    bary, _, mass = oracle.transport_x(X, Y, a, b, f, g, 0.3)
    np.testing.assert_allclose(oracle.apply_plan_x(X, Y, a, b, f, g, 0.3, Y), mass[:, None] * bary, rtol=1e-12)


def _problem(seed, n=6, m=5, d=2):
    rng = np.random.default_rng(seed)
    X = rng.random((n, d))
    Y = rng.random((m, d)) + 0.1
    a = rng.dirichlet(np.ones(n))
    b = rng.dirichlet(np.ones(m))
    return X, Y, a, b


@pytest.mark.parametrize("eps", [0.3, 1.0])
def test_hvp_matches_finite_differences_of_gradient(eps):
    X, Y, a, b = _problem(32)
    V = np.random.default_rng(3).standard_normal(X.shape)

    def grad(X_):
        f, g = oracle.solve(X_, Y, a, b, eps, 3000)
        return oracle.transport_x(X_, Y, a, b, f, g, eps)[1]

    f, g = oracle.solve(X, Y, a, b, eps, 3000)
    hv = oracle.hvp_x(X, Y, a, b, f, g, eps, V)
    h = 1e-5
    fd = (grad(X + h * V) - grad(X - h * V)) / (2 * h)
    np.testing.assert_allclose(hv, fd, rtol=1e-5, atol=1e-7)


def test_hvp_symmetric():
    X, Y, a, b = _problem(33, n=7, m=6, d=3)
    f, g = oracle.solve(X, Y, a, b, 0.2, 3000)
    rng = np.random.default_rng(4)
    U, V = rng.standard_normal(X.shape), rng.standard_normal(X.shape)
    lhs = (U * oracle.hvp_x(X, Y, a, b, f, g, 0.2, V)).sum()
    rhs = (V * oracle.hvp_x(X, Y, a, b, f, g, 0.2, U)).sum()
    assert abs(lhs - rhs) <= 1e-10 * (abs(lhs) + abs(rhs))


def test_hvp_single_target_closed_form():
    X, Y, a, b = _problem(34, n=5, m=1, d=3)
    b = np.ones(1)
    f, g = oracle.solve(X, Y, a, b, 0.1, 5)
    V = np.random.default_rng(5).standard_normal(X.shape)
    np.testing.assert_allclose(oracle.hvp_x(X, Y, a, b, f, g, 0.1, V), 2 * a[:, None] * V, rtol=1e-10)


def test_hvp_large_eps_limit():
    X, Y, a, b = _problem(35, n=5, m=4, d=2)
    eps = 1e7
    f, g = oracle.solve(X, Y, a, b, eps, 5)
    V = np.random.default_rng(6).standard_normal(X.shape)
    np.testing.assert_allclose(oracle.hvp_x(X, Y, a, b, f, g, eps, V), 2 * a[:, None] * b.sum() * V,
                               rtol=1e-5, atol=1e-9)
