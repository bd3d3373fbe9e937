"""GPU parity of the plan application (vector- and matrix-transport products) and
the Hessian-vector product (page "FlashSinkhorn: Trasporto Ottimo Entropico Consapevole delle I/O su GPU",
section "Metodologia", part "3. Differenziazione e Ottimizzazione del Secondo Ordine") against the oracle.

Bounds:
  apply_plan: |d(PV)_ik| <= r_i (rel * max|V_k| (1 + dm) + |avg_ik| dm) with rel = 2e-5
    (fp32) / 5e-4 (bf16) the transport bound of a weighted average, avg = PV/r, and
    dm = expm1(tol_T/eps) the row-mass bound from the half-step.
  hvp: max|dHV| <= tau * max|HV_ref|, tau = 5e-4 (fp32), 5e-3 (bf16).  The HVP
    combines several plan products with weight 2/eps; running the same algorithm in
    fp64 with every plan product perturbed by random relative errors of 1e-6 (1e-5)
    moves the result by 7e-5 (9e-4) relative at eps = 0.1, growing like 1/eps.  The
    plan products carry about 1e-6 (fp32 operands) to 1e-5 (bf16 operands).
Potentials come from converged oracle solves (never from the GPU).
"""

import numpy as np
import pytest
import torch

import oracle
from log_domain_sinkhorn_half_amd import binding as sk
from log_domain_sinkhorn_half_amd.inputs import make_case

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


def potentials(p, eps, iters):
    f, g = oracle.solve(p.X, p.Y, p.a, p.b, eps, iters)
    return f.astype(np.float32), g.astype(np.float32)


def check_apply(p, eps, f, g, side, M, got):
    for k in range(p.batch):
        X, Y, a, b = (np.asarray(v[k], np.float64) for v in (p.X, p.Y, p.a, p.b))
        if side == "x":
            ref = oracle.apply_plan_x(X, Y, a, b, f[k], g[k], eps, M[k])
            mass = oracle.apply_plan_x(X, Y, a, b, f[k], g[k], eps, np.ones(p.m))
            T = oracle.half_step_f(X, Y, b, g[k], eps)
        else:
            ref = oracle.apply_plan_y(X, Y, a, b, f[k], g[k], eps, M[k])
            mass = oracle.apply_plan_y(X, Y, a, b, f[k], g[k], eps, np.ones(p.n))
            T = oracle.half_step_g(X, Y, a, f[k], eps)
        rel = 5e-4 if p.dtype == "bf16" else 2e-5
        tT = 2e-2 * eps if p.dtype == "bf16" else 1e-3 * eps + 1e-5 * float(np.max(np.abs(T)))
        dm = np.expm1(tT / eps)
        avg = np.divide(ref, mass[:, None], out=np.zeros_like(ref), where=mass[:, None] > 0)
        tol = mass[:, None] * (rel * np.max(np.abs(M[k]), axis=0)[None, :] * (1 + dm) + np.abs(avg) * dm)
        err = np.abs(got[k] - ref)
        assert np.all(np.isfinite(got[k]))
        assert np.all(err <= tol), f"apply_{side} problem {k}: worst err {err.max():.3e}, excess {(err - tol).max():.3e}"


@pytest.mark.parametrize("n,m,d,dtype,c", [(300, 200, 3, "fp32", 1), (129, 257, 16, "fp32", 5),
                                           (200, 333, 64, "fp32", 21), (150, 140, 4, "fp32", 70),
                                           (100, 90, 128, "bf16", 7), (63, 65, 8, "bf16", 64),
                                           (40, 50, 88, "fp32", 65), (50, 45, 256, "bf16", 3),
                                           (140, 300, 32, "fp32", 1), (90, 120, 40, "fp32", 30),
                                           # one column: the weighted half-step kernel (bf16 d = 128 and 8,
                                           # fp32 d = 88, and d = 3 past the small-key chunking)
                                           (100, 90, 128, "bf16", 1), (70, 1500, 8, "bf16", 1),
                                           (40, 50, 88, "fp32", 1), (130, 17000, 3, "fp32", 1)])
def test_apply_plan(n, m, d, dtype, c):
    p = make_case(n, m, d, seed=17 * n + c, weights="softmax", dtype=dtype, scale=1.0 / np.sqrt(d))
    eps = 0.1
    f, g = potentials(p, eps, 3)
    rng = np.random.default_rng(c)
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


def test_apply_plan_batched_vector():
    p = make_case(70, 90, 6, batch=3, seed=9, weights="softmax")
    eps = 0.2
    f, g = potentials(p, eps, 3)
    V = np.random.default_rng(4).standard_normal((3, 90)).astype(np.float32)
    X, Y, a, b = dev(p)
    ws = sk.alloc_workspace(X, Y, transport=True)
    sk.init_norms(X, Y, a, b, ws)
    out = sk.apply_plan_x(X, Y, ws, torch.from_numpy(f).cuda(), torch.from_numpy(g).cuda(), eps,
                          torch.from_numpy(V).cuda()).cpu().numpy()
    check_apply(p, eps, f.astype(np.float64), g.astype(np.float64), "x", V[..., None].astype(np.float64),
                out[..., None])


def run_hvp(p, eps, f, g, V, side, iters=400, tol=1e-7):
    X, Y, a, b = dev(p)
    ws = sk.alloc_workspace(X, Y, hvp=True)
    sk.init_norms(X, Y, a, b, ws)
    ft, gt = torch.from_numpy(f).cuda(), torch.from_numpy(g).cuda()
    fn = sk.hvp_x if side == "x" else sk.hvp_y
    out = fn(X, Y, ws, ft, gt, eps, torch.from_numpy(V).cuda(), cg_iters=iters, cg_tol=tol)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("n,m,d,eps,dtype", [(64, 48, 2, 0.5, "fp32"), (200, 150, 3, 0.1, "fp32"),
                                             (120, 140, 16, 0.2, "fp32"), (100, 90, 32, 0.5, "bf16"),
                                             (90, 110, 64, 0.3, "fp32"), (70, 80, 128, 0.5, "bf16"),
                                             (60, 75, 88, 0.4, "fp32"), (50, 60, 256, 0.5, "bf16"),
                                             (80, 100, 32, 0.3, "fp32")])
def test_hvp_against_oracle(n, m, d, eps, dtype):
    p = make_case(n, m, d, seed=23 * n + d, weights="softmax", dtype=dtype, scale=1.0 / np.sqrt(d))
    f, g = potentials(p, eps, 2000)
    rng = np.random.default_rng(d)
    Vx = rng.standard_normal((1, n, d)).astype(np.float32)
    Vy = rng.standard_normal((1, m, d)).astype(np.float32)
    X, Y, a, b = (np.asarray(v[0], np.float64) for v in (p.X, p.Y, p.a, p.b))
    tau = 5e-3 if dtype == "bf16" else 5e-4
    hx = run_hvp(p, eps, f, g, Vx, "x")[0]
    ref_x = oracle.hvp_x(X, Y, a, b, f[0], g[0], eps, Vx[0])
    assert np.max(np.abs(hx - ref_x)) <= tau * np.max(np.abs(ref_x)), np.max(np.abs(hx - ref_x)) / np.max(np.abs(ref_x))
    hy = run_hvp(p, eps, f, g, Vy, "y")[0]
    ref_y = oracle.hvp_x(Y, X, b, a, g[0], f[0], eps, Vy[0])
    assert np.max(np.abs(hy - ref_y)) <= tau * np.max(np.abs(ref_y)), np.max(np.abs(hy - ref_y)) / np.max(np.abs(ref_y))


def test_hvp_symmetric_and_linear_at_larger_size():
    """A property that holds at any size: <U, H V> = <V, H U>, and H is linear."""
    p = make_case(3000, 2500, 3, seed=77, weights="uniform")
    eps = 0.1
    X, Y, a, b = dev(p)
    f, g = sk.solve(X, Y, a, b, eps, 300)
    rng = np.random.default_rng(5)
    U = rng.standard_normal((1, 3000, 3)).astype(np.float32)
    V = rng.standard_normal((1, 3000, 3)).astype(np.float32)
    ws = sk.alloc_workspace(X, Y, hvp=True)
    sk.init_norms(X, Y, a, b, ws)
    hU = sk.hvp_x(X, Y, ws, f, g, eps, torch.from_numpy(U).cuda(), cg_iters=400, cg_tol=1e-7).cpu().numpy()
    hV = sk.hvp_x(X, Y, ws, f, g, eps, torch.from_numpy(V).cuda(), cg_iters=400, cg_tol=1e-7).cpu().numpy()
    W = (2.0 * U - 0.5 * V).astype(np.float32)
    hW = sk.hvp_x(X, Y, ws, f, g, eps, torch.from_numpy(W).cuda(), cg_iters=400, cg_tol=1e-7).cpu().numpy()
    lhs = float((U.astype(np.float64) * hV).sum())
    rhs = float((V.astype(np.float64) * hU).sum())
    scale = float(np.abs(U * hV).sum() + np.abs(V * hU).sum())
    assert abs(lhs - rhs) <= 5e-4 * scale
    lin = 2.0 * hU - 0.5 * hV
    assert np.max(np.abs(hW - lin)) <= 5e-4 * np.max(np.abs(lin))


def test_hvp_batched_problems_are_independent():
    p = make_case(80, 70, 3, batch=3, seed=41, weights="softmax")
    eps = 0.3
    f, g = potentials(p, eps, 2000)
    V = np.random.default_rng(8).standard_normal((3, 80, 3)).astype(np.float32)
    out = run_hvp(p, eps, f, g, V, "x")
    for k in range(3):
        X, Y, a, b = (np.asarray(v[k], np.float64) for v in (p.X, p.Y, p.a, p.b))
        ref = oracle.hvp_x(X, Y, a, b, f[k], g[k], eps, V[k])
        assert np.max(np.abs(out[k] - ref)) <= 5e-4 * np.max(np.abs(ref)), k


def test_transport_and_hvp_are_deterministic():
    p = make_case(500, 400, 3, seed=42, weights="softmax")
    eps = 0.1
    f, g = potentials(p, eps, 5)
    V = np.random.default_rng(9).standard_normal((1, 500, 3)).astype(np.float32)
    h1 = run_hvp(p, eps, f, g, V, "x", iters=30)
    h2 = run_hvp(p, eps, f, g, V, "x", iters=30)
    np.testing.assert_array_equal(h1, h2)
    X, Y, a, b = dev(p)
    ws = sk.alloc_workspace(X, Y, transport=True)
    sk.init_norms(X, Y, a, b, ws)
    ft, gt = torch.from_numpy(f).cuda(), torch.from_numpy(g).cuda()
    b1, g1 = sk.barycentric_x(X, Y, ws, ft, gt, eps)
    b2, g2 = sk.barycentric_x(X, Y, ws, ft, gt, eps)
    assert torch.equal(b1, b2) and torch.equal(g1, g2)


# ---------------------------------------------------------------------------
# HVPs whose conjugate-gradient system spans several 2048-element blocks, against
# the dense oracle (fixture tests/golden/hvp_multiblock.json, written by
# tests/golden/make_hvp_golden.py from the oracle alone)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("side", ["x", "y"])
def test_hvp_multiblock_against_dense_oracle(side):
    import hashlib
    import json
    import os

    path = os.path.join(os.path.dirname(__file__), "golden", "hvp_multiblock.json")
    if not os.path.exists(path):
        pytest.skip("fixture not generated (python tests/golden/make_hvp_golden.py)")
    gold = json.load(open(path))
    case = gold["cases"][side]
    eps = gold["eps"]
    p = make_case(case["n"], case["m"], 3, seed=case["seed"], weights="softmax", eps=eps)
    f, g = oracle.solve(p.X[0], p.Y[0], p.a[0], p.b[0], eps, gold["iters"])
    f, g = f.astype(np.float32), g.astype(np.float32)
    assert hashlib.sha256(f.tobytes() + g.tobytes()).hexdigest()[:16] == case["potentials_sha256_16"]
    rows = p.n if side == "x" else p.m
    V = np.random.default_rng(case["seed"] + 7).standard_normal((rows, 3)).astype(np.float32)
    ref = np.array(case["hv"])
    got = run_hvp(p, eps, f[None], g[None], V[None], side, iters=600, tol=1e-8)[0]
    err = np.max(np.abs(got - ref))
    assert err <= 5e-4 * np.max(np.abs(ref)), err / np.max(np.abs(ref))


# ---------------------------------------------------------------------------
# plan products at the full sizes of the 8192^2 d = 64 (fp32), the 70000^2 d = 3
# (fp32) and the 65536 x 32768 d = 128 (bf16) workloads, on sampled rows computed
# by the oracle one at a time; c = 1, 64 (one pass) and 65 (two passes) columns
# ---------------------------------------------------------------------------
def _sample(n, k, seed):
    rng = np.random.default_rng(seed)
    return np.sort(np.concatenate([rng.choice(n, size=k, replace=False), [0, n - 1]]))


@pytest.mark.parametrize("cfg,c", [(2, 1), (2, 65), (3, 1), (4, 1), (4, 64), (4, 65)])
def test_apply_plan_full_size_sampled_rows(cfg, c):
    from log_domain_sinkhorn_half_amd.inputs import make_config, random_potential

    p = make_config(cfg)
    eps = float(p.eps[-1])
    X, Y, a, b = dev(p)
    ws = sk.alloc_workspace(X, Y, transport=True)
    sk.init_norms(X, Y, a, b, ws)
    Xo, Yo, ao, bo = (np.asarray(v[0], np.float64) for v in (p.X, p.Y, p.a, p.b))
    rng = np.random.default_rng(100 * cfg + c)
    for side in ("x", "y"):
        rows_n, keys_n = (p.n, p.m) if side == "x" else (p.m, p.n)
        R = _sample(rows_n, 48, 7 * cfg + c)
        key_pot = random_potential(keys_n, 50 + cfg, 0.1)
        # the rows' potential: the oracle half-step at the sampled rows (zero elsewhere;
        # those rows' outputs are not checked)
        if side == "x":
            T = oracle.half_step_f(Xo, Yo, bo, key_pot, eps, rows=R)
        else:
            T = oracle.half_step_g(Xo, Yo, ao, key_pot, eps, rows=R)
        row_pot = np.zeros(rows_n, np.float32)
        row_pot[R] = T.astype(np.float32)
        M = rng.standard_normal((keys_n, c)).astype(np.float32)
        f = row_pot if side == "x" else key_pot
        g = key_pot if side == "x" else row_pot
        ft, gt = torch.from_numpy(f[None]).cuda(), torch.from_numpy(g[None]).cuda()
        call = sk.apply_plan_x if side == "x" else sk.apply_plan_y
        got = call(X, Y, ws, ft, gt, eps, torch.from_numpy(M[None]).cuda()).cpu().numpy()[0][R]
        fo, go = f.astype(np.float64), g.astype(np.float64)
        if side == "x":
            ref = oracle.apply_plan_x(Xo, Yo, ao, bo, fo, go, eps, M.astype(np.float64), rows=R)
            mass = oracle.apply_plan_x(Xo, Yo, ao, bo, fo, go, eps, np.ones(keys_n), rows=R)
        else:
            ref = oracle.apply_plan_y(Xo, Yo, ao, bo, fo, go, eps, M.astype(np.float64), rows=R)
            mass = oracle.apply_plan_y(Xo, Yo, ao, bo, fo, go, eps, np.ones(keys_n), rows=R)
        rel = 5e-4 if p.dtype == "bf16" else 2e-5
        tT = 2e-2 * eps if p.dtype == "bf16" else 1e-3 * eps + 1e-5 * float(np.max(np.abs(T)))
        dm = np.expm1(tT / eps)
        avg = ref / mass[:, None]
        tol = mass[:, None] * (rel * np.max(np.abs(M), axis=0)[None, :] * (1 + dm) + np.abs(avg) * dm)
        err = np.abs(got - ref)
        assert np.all(np.isfinite(got)), side
        assert np.all(err <= tol), f"{side}: worst err/tol {(err / tol).max():.3f}"


@pytest.mark.parametrize("c", [1, 65])
def test_apply_plan_full_size_batched_sampled(c):
    """The 64-problem 2048^2 d = 32 workload: one launch over all problems; problems
    0 and 63 checked on sampled rows against the oracle (the others carry zero row
    potentials and are not checked)."""
    from log_domain_sinkhorn_half_amd.inputs import make_config, random_potential

    p = make_config(5)
    eps = float(p.eps[-1])
    X, Y, a, b = dev(p)
    ws = sk.alloc_workspace(X, Y, transport=True)
    sk.init_norms(X, Y, a, b, ws)
    rng = np.random.default_rng(500 + c)
    for side in ("x", "y"):
        rows_n, keys_n = (p.n, p.m) if side == "x" else (p.m, p.n)
        key_pot = np.stack([random_potential(keys_n, 70 + k, 0.1) for k in range(p.batch)]).astype(np.float32)
        row_pot = np.zeros((p.batch, rows_n), np.float32)
        M = rng.standard_normal((p.batch, keys_n, c)).astype(np.float32)
        checks = {}
        for k in (0, p.batch - 1):
            Xo, Yo, ao, bo = (np.asarray(v[k], np.float64) for v in (p.X, p.Y, p.a, p.b))
            R = _sample(rows_n, 40, 11 * k + c)
            if side == "x":
                T = oracle.half_step_f(Xo, Yo, bo, key_pot[k].astype(np.float64), eps, rows=R)
            else:
                T = oracle.half_step_g(Xo, Yo, ao, key_pot[k].astype(np.float64), eps, rows=R)
            row_pot[k, R] = T.astype(np.float32)
            checks[k] = (R, T, Xo, Yo, ao, bo)
        f = row_pot if side == "x" else key_pot
        g = key_pot if side == "x" else row_pot
        call = sk.apply_plan_x if side == "x" else sk.apply_plan_y
        got_all = call(X, Y, ws, torch.from_numpy(f).cuda(), torch.from_numpy(g).cuda(), eps,
                       torch.from_numpy(M).cuda()).cpu().numpy()
        for k, (R, T, Xo, Yo, ao, bo) in checks.items():
            fo, go = f[k].astype(np.float64), g[k].astype(np.float64)
            fn = oracle.apply_plan_x if side == "x" else oracle.apply_plan_y
            ref = fn(Xo, Yo, ao, bo, fo, go, eps, M[k].astype(np.float64), rows=R)
            mass = fn(Xo, Yo, ao, bo, fo, go, eps, np.ones(keys_n), rows=R)
            tT = 1e-3 * eps + 1e-5 * float(np.max(np.abs(T)))
            dm = np.expm1(tT / eps)
            avg = ref / mass[:, None]
            tol = mass[:, None] * (2e-5 * np.max(np.abs(M[k]), axis=0)[None, :] * (1 + dm) + np.abs(avg) * dm)
            got = got_all[k][R]
            err = np.abs(got - ref)
            assert np.all(np.isfinite(got)), (side, k)
            assert np.all(err <= tol), f"{side} problem {k}: worst err/tol {(err / tol).max():.3f}"


@pytest.mark.parametrize("cfg,lin_tol", [(2, 1e-3), (3, 1e-4), (4, 2e-3)])
def test_hvp_full_size_symmetric_and_linear(cfg, lin_tol):
    """Properties that hold at any size, at the 8192^2 d = 64, 70000^2 d = 3 and
    65536 x 32768 d = 128 (bf16, annealed) workloads: after the workload's own solve,
    <U, H V> = <V, H U> and H(2U - V/2) = 2 HU - HV/2 (CG to 1e-7).  Measured: symmetric
    to about 1e-8, linear to 8e-5, 3e-6 and 3.4e-4 relative."""
    from log_domain_sinkhorn_half_amd.inputs import make_config

    p = make_config(cfg)
    X, Y, a, b = dev(p)
    sched = [float(e) for e in p.eps]
    if len(sched) > 1:
        f, g = sk.solve(X, Y, a, b, sched, len(sched))
    else:
        f, g = sk.solve(X, Y, a, b, sched[0], p.iters)
    eps = sched[-1]
    rng = np.random.default_rng(cfg)
    U = rng.standard_normal((1, p.n, p.d)).astype(np.float32)
    V = rng.standard_normal((1, p.n, p.d)).astype(np.float32)
    W = (2.0 * U - 0.5 * V).astype(np.float32)
    ws = sk.alloc_workspace(X, Y, hvp=True)
    sk.init_norms(X, Y, a, b, ws)
    h = {}
    for nm, A in (("U", U), ("V", V), ("W", W)):
        h[nm] = sk.hvp_x(X, Y, ws, f, g, eps, torch.from_numpy(A).cuda(), cg_iters=400,
                         cg_tol=1e-7).cpu().numpy().astype(np.float64)
    assert all(np.all(np.isfinite(v)) for v in h.values())
    lhs = float((U[0] * h["V"][0]).sum())
    rhs = float((V[0] * h["U"][0]).sum())
    scale = float(np.abs(U[0] * h["V"][0]).sum() + np.abs(V[0] * h["U"][0]).sum())
    assert abs(lhs - rhs) <= 1e-6 * scale, abs(lhs - rhs) / scale
    lin = 2.0 * h["U"][0] - 0.5 * h["V"][0]
    rel = np.max(np.abs(h["W"][0] - lin)) / np.max(np.abs(lin))
    assert rel <= lin_tol, rel

