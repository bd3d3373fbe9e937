"""GPU parity of the wide plan passes (transport, plan application and HVP for fp32
inputs with d > 88 and bf16 inputs with d > 256) against the fp64 oracle, up to
d = 1024 (page "FlashSinkhorn: Trasporto Ottimo Entropico Consapevole delle I/O su GPU",
section "Risultati Sperimentali" for the widths; section "Metodologia", part
"3. Differenziazione e Ottimizzazione del Secondo Ordine" for the operations).

These passes take the rows' half-step, write the weights of a block of rows
against all keys as bf16 hi/lo parts (2^-17 relative), and multiply them with
the value rows (fp32 coordinates in two bf16 parts, 2^-17 relative; bf16 ones
exact; matrix columns in three parts, exact).

Bounds on the weighted averages (bary, and plan products divided by the row mass):
  fp32 (hi/lo scores): the base-2 score of row i carries at most
      ds_i = 2 lambda (2^-16 + 4 sqrt(3d) 2^-24) |x_i - c| max_j |y_j - c|
  (per coordinate the three bf16 products x_h v_h + x_h v_l + x_l v_h drop terms
  below 0.75 * 2^-16 |x_t v_t|; the fp32 sum of 3d products is taken at four times
  its probabilistic sqrt(n) u size (Higham and Mary, "A new approach to
  probabilistic rounding error analysis", 2019); c is the joint bounding-box
  centre, which the library subtracts).  Every weight then moves by a factor
  within exp(+-eta), eta = ln2 ds_i + 2^-17 (its hi/lo split), so a normalised
  average moves by at most expm1(2 eta) times the weighted mean deviation, which
  Cauchy-Schwarz bounds by the weighted standard deviation sd_it (from the
  oracle's plan), plus 2^-17 max_j |y_jt - c_t| for the two value parts.
  (Measured: at most 3% of this bound, except where a row has a single key and
  the value parts are the whole error.)
  bf16: the transport bound 5e-4 max|V| widened by (d/8 + 2)/18 past d = 128.
  grad and plan products: as in the narrow tests, with the half-step bound tol_T
  (1e-3 eps + 1e-5 max|T| fp32, 2e-2 eps bf16) for the row mass.
  hvp: tau max|HV_ref| with the narrow tests' tau, 5e-4 (fp32) and 5e-3 (bf16): the
  HVP amplifies plan-product errors about 100-fold at these eps (measured at most
  2.1e-5 relative for fp32 and 1.0e-4 for bf16 at d = 1024).
Potentials come from the oracle, never from the HIP path.
"""

import numpy as np
import pytest
import torch

import oracle
from log_domain_sinkhorn_half_amd import binding as sk
from log_domain_sinkhorn_half_amd.inputs import make_case, random_potential

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sk.load_library()


def dev(p):
    if p.dtype == "bf16":
        X = torch.from_numpy(p.X_bits.view(np.int16)).cuda().view(torch.bfloat16)
        Y = torch.from_numpy(p.Y_bits.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        X = torch.from_numpy(p.X).cuda()
        Y = torch.from_numpy(p.Y).cuda()
    return X, Y, torch.from_numpy(p.a).cuda(), torch.from_numpy(p.b).cuda()


def score_eta(p, eps, P, V):
    """Per-row bound eta_i on the natural-log error of a weight (fp32 hi/lo path)."""
    both = np.concatenate([P, V])
    c = 0.5 * (both.min(0) + both.max(0))
    rp = np.sqrt(((P - c) ** 2).sum(1))
    rv = float(np.sqrt(((V - c) ** 2).sum(1)).max())
    lam = np.log2(np.e) / eps
    ds = 2 * lam * (2.0 ** -16 + 4 * np.sqrt(3 * p.d) * 2.0 ** -24) * rp * rv
    return np.log(2) * ds + 2.0 ** -17, c


def avg_bound(p, eps, P, V, sd, rows=None):
    """Bound on each coordinate of a weighted average of the rows of V (keys) for
    the queries P[rows], sd the weighted standard deviations [rows, d]."""
    if p.dtype == "bf16":
        return np.full(sd.shape, 5e-4 * (p.d / 8 + 2) / 18 * float(np.max(np.abs(V))))
    eta, c = score_eta(p, eps, P, V)
    eta = eta if rows is None else eta[rows]
    return np.expm1(2 * eta)[:, None] * sd + 2.0 ** -17 * np.max(np.abs(V - c), axis=0)[None, :]


def half_tol(p, eps, T):
    return 2e-2 * eps if p.dtype == "bf16" else 1e-3 * eps + 1e-5 * float(np.max(np.abs(T)))


def check_transport(p, k, side, eps, bary, grad, f, g, rows=None):
    X, Y, a, b = (np.asarray(v[k], np.float64) for v in (p.X, p.Y, p.a, p.b))
    if side == "x":
        P, V, T = X, Y, oracle.half_step_f(X, Y, b, g[k], eps, rows=rows)
        bary_ref, grad_ref, mass = oracle.transport_x(X, Y, a, b, f[k], g[k], eps, rows=rows)
    else:
        P, V, T = Y, X, oracle.half_step_g(X, Y, a, f[k], eps, rows=rows)
        bary_ref, grad_ref, mass = oracle.transport_y(X, Y, a, b, f[k], g[k], eps, rows=rows)
    Psel = P if rows is None else P[rows]
    got_b = bary[k] if rows is None else bary[k][rows]
    got_g = grad[k] if rows is None else grad[k][rows]
    # weighted standard deviation of the values per row and coordinate
    if side == "x":
        m2 = oracle.apply_plan_x(X, Y, a, b, f[k], g[k], eps, Y ** 2, rows=rows)
    else:
        m2 = oracle.apply_plan_y(X, Y, a, b, f[k], g[k], eps, X ** 2, rows=rows)
    with np.errstate(invalid="ignore", divide="ignore"):
        var = np.where(mass[:, None] > 0, m2 / mass[:, None] - bary_ref ** 2, 0.0)
    sd = np.sqrt(np.maximum(var, 0.0))
    tb = avg_bound(p, eps, P, V, sd, rows)
    assert np.all(np.isfinite(got_b)) and np.all(np.isfinite(got_g))
    err = np.abs(got_b - bary_ref)
    worst = float(np.max(err / tb))
    assert worst <= 1.0, f"bary_{side} d={p.d}: max err {err.max():.3e}, worst err/bound {worst:.3f}"
    dm = np.expm1(half_tol(p, eps, T) / eps)
    tg = 2.0 * mass[:, None] * (tb * (1.0 + dm) + np.abs(Psel - bary_ref) * dm)
    excess = np.abs(got_g - grad_ref) - tg
    assert np.all(excess <= 0), f"grad_{side} d={p.d}: worst excess {excess.max():.3e}"
    return err.max(), worst


def run_transport(p, f, g, eps):
    X, Y, a, b = dev(p)
    ws = sk.alloc_workspace(X, Y, transport=True)
    sk.init_norms(X, Y, a, b, ws)
    ft = torch.from_numpy(np.asarray(f, np.float32)).cuda()
    gt = torch.from_numpy(np.asarray(g, np.float32)).cuda()
    bx, gx = sk.barycentric_x(X, Y, ws, ft, gt, eps)
    by, gy = sk.barycentric_y(X, Y, ws, ft, gt, eps)
    torch.cuda.synchronize()
    flags = sk.range_flags(X, Y, ws)
    return bx.cpu().numpy(), gx.cpu().numpy(), by.cpu().numpy(), gy.cpu().numpy(), flags


def oracle_potentials(p, eps, iters=3):
    f, g = oracle.solve(p.X, p.Y, p.a, p.b, eps, iters)
    return f.astype(np.float32).astype(np.float64), g.astype(np.float32).astype(np.float64)


@pytest.mark.parametrize("n,m,d,dtype", [(300, 200, 89, "fp32"), (257, 300, 128, "fp32"), (200, 513, 512, "fp32"),
                                         (90, 70, 1024, "fp32"), (1, 7, 100, "fp32"), (130, 260, 300, "bf16"),
                                         (300, 129, 512, "bf16"), (70, 90, 1024, "bf16")])
def test_transport_wide(n, m, d, dtype):
    p = make_case(n, m, d, seed=7 * n + d, weights="softmax", dtype=dtype, scale=1.0 / np.sqrt(d))
    for eps in (0.5, 0.05):
        f, g = oracle_potentials(p, eps)
        bx, gx, by, gy, flags = run_transport(p, f, g, eps)
        ex = check_transport(p, 0, "x", eps, bx, gx, f, g)
        ey = check_transport(p, 0, "y", eps, by, gy, f, g)
        print(f"d={d} {dtype} eps={eps}: bary max err (err/bound) x {ex[0]:.2e} ({ex[1]:.3f}) "
              f"y {ey[0]:.2e} ({ey[1]:.3f})")
        assert flags == 0


def test_transport_wide_batched():
    p = make_case(150, 180, 160, batch=3, seed=4, weights="softmax", scale=1.0 / np.sqrt(160))
    eps = 0.1
    f, g = oracle_potentials(p, eps)
    bx, gx, by, gy, _ = run_transport(p, f, g, eps)
    for k in range(3):
        check_transport(p, k, "x", eps, bx, gx, f, g)
        check_transport(p, k, "y", eps, by, gy, f, g)


def test_transport_wide_several_row_blocks():
    """12000 rows against 50000 keys: the 1 GiB weights buffer holds 5120 rows, so
    the pass runs in three row blocks (the last one ragged); oracle on sampled rows."""
    n, m, d = 12000, 50000, 130
    p = make_case(n, m, d, seed=77, weights="softmax", scale=1.0 / np.sqrt(d))
    eps = 0.1
    rng = np.random.default_rng(78)
    rows = np.unique(np.concatenate([rng.choice(n, 40, replace=False), [0, 5119, 5120, 10239, 10240, n - 1]]))
    X, Y, a, b = (np.asarray(v[0], np.float64) for v in (p.X, p.Y, p.a, p.b))
    g = random_potential((1, m), 79, 0.1).astype(np.float64)
    f = random_potential((1, n), 80, 0.1).astype(np.float64)
    f[0, rows] = oracle.half_step_f(X, Y, b, g[0], eps, rows=rows).astype(np.float32)
    Xt, Yt, at, bt = dev(p)
    ws = sk.alloc_workspace(Xt, Yt, transport=True)
    sk.init_norms(Xt, Yt, at, bt, ws)
    bx, gx = sk.barycentric_x(Xt, Yt, ws, torch.from_numpy(f.astype(np.float32)).cuda(),
                              torch.from_numpy(g.astype(np.float32)).cuda(), eps)
    torch.cuda.synchronize()
    check_transport(p, 0, "x", eps, bx.cpu().numpy(), gx.cpu().numpy(), f, g, rows=rows)


def check_apply(p, eps, f, g, side, M, got):
    X, Y, a, b = (np.asarray(v[0], np.float64) for v in (p.X, p.Y, p.a, p.b))
    if side == "x":
        ref = oracle.apply_plan_x(X, Y, a, b, f[0], g[0], eps, M[0])
        mass = oracle.apply_plan_x(X, Y, a, b, f[0], g[0], eps, np.ones(p.m))
        T = oracle.half_step_f(X, Y, b, g[0], eps)
        P, Q = X, Y
    else:
        ref = oracle.apply_plan_y(X, Y, a, b, f[0], g[0], eps, M[0])
        mass = oracle.apply_plan_y(X, Y, a, b, f[0], g[0], eps, np.ones(p.n))
        T = oracle.half_step_g(X, Y, a, f[0], eps)
        P, Q = Y, X
    # a weighted average of a matrix column moves by at most expm1(2 eta) times
    # its largest deviation, 2 max|M_k| (the three parts of M are exact)
    if p.dtype == "bf16":
        rel = np.full(P.shape[0], 2 * 5e-4 * (p.d / 8 + 2) / 18)
    else:
        rel = 2 * np.expm1(2 * score_eta(p, eps, P, Q)[0]) + 1e-6
    dm = np.expm1(half_tol(p, eps, T) / eps)
    avg = np.divide(ref, mass[:, None], out=np.zeros_like(ref), where=mass[:, None] > 0)
    tol = mass[:, None] * (rel[:, None] * np.max(np.abs(M[0]), axis=0)[None, :] * (1 + dm) + np.abs(avg) * dm)
    err = np.abs(got[0] - ref)
    assert np.all(np.isfinite(got[0]))
    assert np.all(err <= tol), f"apply_{side} d={p.d}: worst err {err.max():.3e}, excess {(err - tol).max():.3e}"


@pytest.mark.parametrize("n,m,d,dtype,c", [(200, 150, 100, "fp32", 1), (129, 257, 200, "fp32", 65),
                                           (150, 140, 100, "fp32", 150), (100, 90, 300, "bf16", 64),
                                           (90, 120, 512, "bf16", 1), (60, 50, 1024, "fp32", 3)])
def test_apply_plan_wide(n, m, d, dtype, c):
    """c = 150 at d = 100 takes three column passes (69 matrix columns each)."""
    p = make_case(n, m, d, seed=31 * n + c, weights="softmax", dtype=dtype, scale=1.0 / np.sqrt(d))
    eps = 0.1
    f, g = oracle.solve(p.X, p.Y, p.a, p.b, eps, 3)
    f, g = f.astype(np.float32), g.astype(np.float32)
    rng = np.random.default_rng(c + d)
    Vx = rng.standard_normal((1, m, c)).astype(np.float32)
    Uy = rng.standard_normal((1, n, c)).astype(np.float32)
    X, Y, a, b = dev(p)
    ws = sk.alloc_workspace(X, Y, transport=True)
    sk.init_norms(X, Y, a, b, ws)
    ft, gt = torch.from_numpy(f).cuda(), torch.from_numpy(g).cuda()
    ox = sk.apply_plan_x(X, Y, ws, ft, gt, eps, torch.from_numpy(Vx).cuda()).cpu().numpy()
    oy = sk.apply_plan_y(X, Y, ws, ft, gt, eps, torch.from_numpy(Uy).cuda()).cpu().numpy()
    check_apply(p, eps, f.astype(np.float64), g.astype(np.float64), "x", Vx.astype(np.float64), ox)
    check_apply(p, eps, f.astype(np.float64), g.astype(np.float64), "y", Uy.astype(np.float64), oy)


@pytest.mark.parametrize("n,m,d,eps,dtype", [(60, 75, 100, 0.4, "fp32"), (50, 45, 300, 0.5, "fp32"),
                                             (50, 60, 300, 0.5, "bf16"), (40, 35, 1024, 0.5, "bf16")])
def test_hvp_wide(n, m, d, eps, dtype):
    p = make_case(n, m, d, seed=41 * n + d, weights="softmax", dtype=dtype, scale=1.0 / np.sqrt(d))
    f, g = oracle.solve(p.X, p.Y, p.a, p.b, eps, 2000)
    f, g = f.astype(np.float32), g.astype(np.float32)
    rng = np.random.default_rng(d + 1)
    Vx = rng.standard_normal((1, n, d)).astype(np.float32)
    Vy = rng.standard_normal((1, m, d)).astype(np.float32)
    X, Y, a, b = (np.asarray(v[0], np.float64) for v in (p.X, p.Y, p.a, p.b))
    tau = 5e-3 if dtype == "bf16" else 5e-4
    Xt, Yt, at, bt = dev(p)
    ws = sk.alloc_workspace(Xt, Yt, hvp=True)
    sk.init_norms(Xt, Yt, at, bt, ws)
    ft, gt = torch.from_numpy(f).cuda(), torch.from_numpy(g).cuda()
    hx = sk.hvp_x(Xt, Yt, ws, ft, gt, eps, torch.from_numpy(Vx).cuda(), cg_iters=400, cg_tol=1e-7)
    hy = sk.hvp_y(Xt, Yt, ws, ft, gt, eps, torch.from_numpy(Vy).cuda(), cg_iters=400, cg_tol=1e-7)
    torch.cuda.synchronize()
    ref_x = oracle.hvp_x(X, Y, a, b, f[0], g[0], eps, Vx[0])
    ref_y = oracle.hvp_x(Y, X, b, a, g[0], f[0], eps, Vy[0])
    for got, ref, side in ((hx.cpu().numpy()[0], ref_x, "x"), (hy.cpu().numpy()[0], ref_y, "y")):
        rel = np.max(np.abs(got - ref)) / np.max(np.abs(ref))
        print(f"hvp_{side} d={d} {dtype}: relative err {rel:.2e}")
        assert rel <= tau, f"hvp_{side} d={d}: relative err {rel:.3e} > {tau:.1e}"
