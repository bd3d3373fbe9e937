"""fp64 CPU oracle for log-domain Sinkhorn (squared-Euclidean cost).

TEST INFRASTRUCTURE.  Only ``tests/``, the smoke check in ``__graft_entry__``
and the CPU-baseline leg of ``bench.py`` may import this package.  The HIP
library never calls it and shares no code with it.

The arithmetic lives in ``sinkhorn_oracle.c`` (plain loops, fp64, OpenMP over
rows); this module compiles it with gcc and wraps it with ctypes.  Inputs are
converted to float64 copies of whatever values the caller passes (for bf16
problems: the exact bf16 values).

Method (page "FlashSinkhorn: Trasporto Ottimo Entropico Consapevole delle I/O su GPU", section
"Metodologia", part "1. Riformulazione in Forma di Attenzione"): f_i <- -eps LSE_j[(g_j - C_ij)/eps
+ log b_j] with
C_ij = ||x_i - y_j||^2, then the mirrored update for g with the new f.

Parity status of each function:
  half_step / half_step_f / half_step_g : pinned (plan marginals after a
      half-step, m=1 and n=1 closed forms, large-eps expansion, symmetry)
  solve            : pinned (gauge shift, dual ascent, eps->0 assignment limit,
                     invariances, fixed points of the closed forms)
  plan_marginals   : pinned (closed forms; numpy brute force in the tests)
  transport / transport_x / transport_y : pinned (m=1 closed form, large-eps
      weighted mean, eps->0 assignment limit, finite differences of the
      converged dual value, translation balance of the two gradients,
      numpy brute force on tiny inputs)
  apply_plan_x / apply_plan_y : pinned (dense numpy plan; equals mass * bary
      for V = the other cloud)
  hvp_x            : pinned (central finite differences of the converged
      gradient along the direction; symmetry of the Hessian; zero for a common
      translation of both clouds in the joint form)
  normalize / cosine_grad : pinned (cost = 2 - 2 cos of the angle in closed
      form for d = 2, invariance of the potentials under positive rescaling of
      points, finite differences of the converged dual value in the raw points,
      gradient orthogonal to its point)
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sinkhorn_oracle.c")
_LIB = os.path.join(_HERE, "_sinkhorn_oracle.so")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I64 = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, IEEE semantics: no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    lib.oracle_threads.argtypes = [ctypes.c_int]
    lib.oracle_threads.restype = ctypes.c_int
    lib.oracle_half_step.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _D, _D, _D,
                                     _D, ctypes.c_double, _I64, ctypes.c_int64, _D, ctypes.c_int]
    lib.oracle_half_step.restype = None
    lib.oracle_solve.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _D, _D, _D, _D,
                                 _D, ctypes.c_int64, ctypes.c_int64, _D, _D, ctypes.c_int]
    lib.oracle_solve.restype = None
    lib.oracle_plan_marginals.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _D, _D,
                                          _D, _D, _D, _D, ctypes.c_double, _D, _D, ctypes.c_int]
    lib.oracle_plan_marginals.restype = None
    lib.oracle_transport.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _D, _D, _D, _D,
                                     _D, _D, ctypes.c_double, _I64, ctypes.c_int64, _D, _D, _D,
                                     ctypes.c_int]
    lib.oracle_transport.restype = None
    lib.oracle_apply_plan.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _D, _D, _D, _D,
                                      _D, _D, ctypes.c_double, _D, ctypes.c_int64, _I64, ctypes.c_int64,
                                      _D, ctypes.c_int]
    lib.oracle_apply_plan.restype = None
    _lib = lib
    return lib


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(x: np.ndarray):
    return x.ctypes.data_as(_D)


def threads_used(threads: Optional[int] = None) -> int:
    """Threads the oracle's parallel loops use for a request (None = default)."""
    return int(_load().oracle_threads(int(threads or 0)))


def half_step(P, Q, w, h, eps: float, rows=None, threads: Optional[int] = None) -> np.ndarray:
    """out[r] = -eps * LSE_j[(h_j - ||P[rows[r]] - Q_j||^2)/eps + log w_j] (2-D inputs)."""
    lib = _load()
    P, Q, w, h = _f64(P), _f64(Q), _f64(w), _f64(h)
    np_, d = P.shape
    nq = Q.shape[0]
    assert Q.shape[1] == d and w.shape == (nq,) and h.shape == (nq,)
    if rows is None:
        out = np.empty(np_, dtype=np.float64)
        lib.oracle_half_step(np_, nq, d, _ptr(P), _ptr(Q), _ptr(w), _ptr(h), float(eps),
                             None, np_, _ptr(out), int(threads or 0))
    else:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        assert rows.ndim == 1 and (rows.size == 0 or (rows.min() >= 0 and rows.max() < np_))
        out = np.empty(rows.size, dtype=np.float64)
        lib.oracle_half_step(np_, nq, d, _ptr(P), _ptr(Q), _ptr(w), _ptr(h), float(eps),
                             rows.ctypes.data_as(_I64), rows.size, _ptr(out), int(threads or 0))
    return out


def half_step_f(X, Y, b, g, eps: float, rows=None, threads=None) -> np.ndarray:
    """f_i = -eps LSE_j[(g_j - C_ij)/eps + log b_j] for one problem ([n,d], [m,d])."""
    return half_step(X, Y, b, g, eps, rows=rows, threads=threads)


def half_step_g(X, Y, a, f, eps: float, rows=None, threads=None) -> np.ndarray:
    """g_j = -eps LSE_i[(f_i - C_ij)/eps + log a_i] for one problem ([n,d], [m,d])."""
    return half_step(Y, X, a, f, eps, rows=rows, threads=threads)


def solve(X, Y, a, b, eps, iters: int, g0=None, threads: Optional[int] = None):
    """Run `iters` alternating iterations (f then g) from g = g0 (default 0).

    Accepts single ([n,d]) or batched ([B,n,d]) problems; eps is a scalar or an
    array of length iters (a per-iteration schedule).  Returns fp64 (f, g).
    """
    lib = _load()
    X, Y, a, b = _f64(X), _f64(Y), _f64(a), _f64(b)
    batched = X.ndim == 3
    if not batched:
        X, Y, a, b = X[None], Y[None], a[None], b[None]
    B, n, d = X.shape
    m = Y.shape[1]
    e = np.atleast_1d(_f64(eps))
    assert e.size in (1, iters)
    f = np.zeros((B, n), dtype=np.float64)
    g = np.zeros((B, m), dtype=np.float64) if g0 is None else _f64(np.broadcast_to(g0, (B, m))).copy()
    for p in range(B):
        Xp, Yp = np.ascontiguousarray(X[p]), np.ascontiguousarray(Y[p])
        ap, bp = np.ascontiguousarray(a[p]), np.ascontiguousarray(b[p])
        fp, gp = np.ascontiguousarray(f[p]), np.ascontiguousarray(g[p])
        lib.oracle_solve(n, m, d, _ptr(Xp), _ptr(Yp), _ptr(ap), _ptr(bp), _ptr(e), e.size,
                         int(iters), _ptr(fp), _ptr(gp), int(threads or 0))
        f[p], g[p] = fp, gp
    if not batched:
        return f[0], g[0]
    return f, g


def plan_marginals(X, Y, a, b, f, g, eps: float, threads: Optional[int] = None):
    """Row and column sums of P_ij = a_i b_j exp((f_i + g_j - C_ij)/eps)."""
    lib = _load()
    X, Y, a, b, f, g = (_f64(v) for v in (X, Y, a, b, f, g))
    n, d = X.shape
    m = Y.shape[0]
    row = np.empty(n, dtype=np.float64)
    col = np.empty(m, dtype=np.float64)
    lib.oracle_plan_marginals(n, m, d, _ptr(X), _ptr(Y), _ptr(a), _ptr(b), _ptr(f), _ptr(g),
                              float(eps), _ptr(row), _ptr(col), int(threads or 0))
    return row, col


def marginal_error(X, Y, a, b, f, g, eps: float, threads: Optional[int] = None):
    """L1 deviations (sum_i |row_i - a_i|, sum_j |col_j - b_j|) of the plan's marginals."""
    row, col = plan_marginals(X, Y, a, b, f, g, eps, threads=threads)
    return float(np.abs(row - _f64(a)).sum()), float(np.abs(col - _f64(b)).sum())


def transport(P, Q, wp, wq, hp, hq, eps: float, rows=None, threads: Optional[int] = None):
    """Barycentric projection, gradient and row mass of the plan
    pi_rj = wp_r wq_j exp((hp_r + hq_j - ||P_r - Q_j||^2)/eps) for the rows of P.

    Returns (bary [k,d], grad [k,d], mass [k]) for the selected rows (all by default):
    bary_r = sum_j pi_rj Q_j / sum_j pi_rj, grad_r = sum_j pi_rj 2 (P_r - Q_j),
    mass_r = sum_j pi_rj.
    """
    lib = _load()
    P, Q, wp, wq, hp, hq = (_f64(v) for v in (P, Q, wp, wq, hp, hq))
    np_, d = P.shape
    nq = Q.shape[0]
    assert Q.shape[1] == d and wp.shape == (np_,) and hp.shape == (np_,)
    assert wq.shape == (nq,) and hq.shape == (nq,)
    if rows is None:
        k, rp = np_, None
    else:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        assert rows.ndim == 1 and (rows.size == 0 or (rows.min() >= 0 and rows.max() < np_))
        k, rp = rows.size, rows.ctypes.data_as(_I64)
    bary = np.empty((k, d), dtype=np.float64)
    grad = np.empty((k, d), dtype=np.float64)
    mass = np.empty(k, dtype=np.float64)
    lib.oracle_transport(np_, nq, d, _ptr(P), _ptr(Q), _ptr(wp), _ptr(wq), _ptr(hp), _ptr(hq),
                         float(eps), rp, k, _ptr(bary), _ptr(grad), _ptr(mass), int(threads or 0))
    return bary, grad, mass


def transport_x(X, Y, a, b, f, g, eps: float, rows=None, threads=None):
    """Transport application for the points of X: bary_i = (P Y)_i / (P 1)_i,
    grad_i = sum_j P_ij 2 (x_i - y_j), mass_i = (P 1)_i, P_ij = a_i b_j exp((f_i + g_j - C_ij)/eps)."""
    return transport(X, Y, a, b, f, g, eps, rows=rows, threads=threads)


def transport_y(X, Y, a, b, f, g, eps: float, rows=None, threads=None):
    """Transport application for the points of Y (the same plan read by columns):
    bary_j = (P^T X)_j / (P^T 1)_j, grad_j = sum_i P_ij 2 (y_j - x_i), mass_j = (P^T 1)_j."""
    return transport(Y, X, b, a, g, f, eps, rows=rows, threads=threads)


# ---------------------------------------------------------------------------
# Cosine cost (page "FlashSinkhorn: Trasporto Ottimo Entropico Consapevole delle I/O su GPU",
# section "Significato e Affermazioni": the method covers squared-Euclidean cost and the cosine
# distance
# after normalisation).  C_ij = ||x_i/|x_i| - y_j/|y_j|||^2 = 2 - 2 cos(x_i, y_j);
# a zero point stays zero.  Every routine above applies unchanged to the
# normalised clouds; only the gradient in the raw points needs the chain rule.
# ---------------------------------------------------------------------------
def normalize(P) -> np.ndarray:
    """Rows of P divided by their Euclidean norm (fp64); zero rows stay zero."""
    P = _f64(P)
    nrm = np.sqrt((P * P).sum(-1, keepdims=True))
    return np.divide(P, nrm, out=np.zeros_like(P), where=nrm > 0)


def cosine_grad(P, grad_hat) -> np.ndarray:
    """Gradient in the raw points from the gradient in the normalised points:
    d(p/|p|)/dp = (I - p_hat p_hat^T)/|p|, applied row by row (zero rows: 0)."""
    P, G = _f64(P), _f64(grad_hat)
    out = np.zeros_like(P)
    for i in range(P.shape[0]):
        nrm = float(np.sqrt(P[i] @ P[i]))
        if nrm > 0:
            ph = P[i] / nrm
            out[i] = (G[i] - (ph @ G[i]) * ph) / nrm
    return out


def apply_plan(P, Q, wp, wq, hp, hq, eps: float, V, rows=None, threads: Optional[int] = None) -> np.ndarray:
    """out_r = sum_j pi_rj V_j with pi_rj = wp_r wq_j exp((hp_r + hq_j - ||P_r - Q_j||^2)/eps)."""
    lib = _load()
    P, Q, wp, wq, hp, hq = (_f64(v) for v in (P, Q, wp, wq, hp, hq))
    V = _f64(V)
    squeeze = V.ndim == 1
    if squeeze:
        V = V[:, None].copy()
    np_, d = P.shape
    nq, c = V.shape
    assert Q.shape == (nq, d)
    if rows is None:
        k, rp = np_, None
    else:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        k, rp = rows.size, rows.ctypes.data_as(_I64)
    out = np.empty((k, c), dtype=np.float64)
    lib.oracle_apply_plan(np_, nq, d, _ptr(P), _ptr(Q), _ptr(wp), _ptr(wq), _ptr(hp), _ptr(hq), float(eps),
                          _ptr(V), c, rp, k, _ptr(out), int(threads or 0))
    return out[:, 0] if squeeze else out


def apply_plan_x(X, Y, a, b, f, g, eps: float, V, rows=None, threads=None):
    """(P V)_i = sum_j P_ij V_j, V: [m] or [m, c]."""
    return apply_plan(X, Y, a, b, f, g, eps, V, rows=rows, threads=threads)


def apply_plan_y(X, Y, a, b, f, g, eps: float, U, rows=None, threads=None):
    """(P^T U)_j = sum_i P_ij U_i, U: [n] or [n, c]."""
    return apply_plan(Y, X, b, a, g, f, eps, U, rows=rows, threads=threads)


def hvp_x(X, Y, a, b, f, g, eps: float, V) -> np.ndarray:
    """Hessian of the entropic OT value in the points X, applied to the direction V
    (page "FlashSinkhorn: Trasporto Ottimo Entropico Consapevole delle I/O su GPU", section
    "Metodologia", part "3. Differenziazione e Ottimizzazione del Secondo Ordine": Hessian-vector
    products without the Hessian).

    Plain dense definition for small problems, at potentials (f, g) taken as optimal:
    the gradient is G_i = sum_j P_ij 2 (x_i - y_j).  Moving X along V moves the cost by
    dC_ij = 2 (x_i - y_j) . v_i and the potentials by (df, dg), which keep the plan's
    marginals fixed:  sum_j P_ij (df_i + dg_j - dC_ij) = 0 for every i and
    sum_i P_ij (df_i + dg_j - dC_ij) = 0 for every j  (solved here by least squares on
    the full (n+m) system; its null direction (1, -1) does not change the plan).  Then
    dP = P * (df + dg - dC)/eps and  H V = sum_j dP_ij 2 (x_i - y_j) + 2 (sum_j P_ij) v_i.
    """
    X, Y, a, b, f, g, V = (_f64(v) for v in (X, Y, a, b, f, g, V))
    n, m = X.shape[0], Y.shape[0]
    D = X[:, None, :] - Y[None, :, :]                      # x_i - y_j
    C = (D * D).sum(-1)
    P = a[:, None] * b[None, :] * np.exp((f[:, None] + g[None, :] - C) / eps)
    dC = 2.0 * (D * V[:, None, :]).sum(-1)
    A = np.zeros((n + m, n + m))
    A[:n, :n] = np.diag(P.sum(1))
    A[:n, n:] = P
    A[n:, :n] = P.T
    A[n:, n:] = np.diag(P.sum(0))
    rhs = np.concatenate([(P * dC).sum(1), (P * dC).sum(0)])
    sol = np.linalg.lstsq(A, rhs, rcond=None)[0]
    df, dg = sol[:n], sol[n:]
    dP = P * (df[:, None] + dg[None, :] - dC) / eps
    return 2.0 * (dP[:, :, None] * D).sum(1) + 2.0 * P.sum(1)[:, None] * V
