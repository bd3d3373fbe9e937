"""GPU: translated clouds and the score-range contract, against the fp64 oracle.

The squared-Euclidean cost is translation-invariant, so the library centres both
clouds on one common vector before forming norms and operands.  Far from the
origin the potentials then keep the fp32 (bf16) bounds; the oracle forms each
cost from coordinate differences of the translated values themselves.  Scores
beyond the supported range must be reported in the workspace's status word.
"""

import numpy as np
import pytest
import torch

import oracle
from log_domain_sinkhorn_half_amd import binding as sk
from log_domain_sinkhorn_half_amd.inputs import make_case, make_config, random_potential, translate

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
        X, Y = torch.from_numpy(p.X).cuda(), torch.from_numpy(p.Y).cuda()
    return X, Y, torch.from_numpy(p.a).cuda(), torch.from_numpy(p.b).cuda()


def bound(p, eps, ref):
    if p.dtype == "bf16":
        return 2e-2 * eps
    return 1e-3 * eps + 1e-5 * float(np.max(np.abs(ref)))


def check(got, ref, b, what):
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = float(np.max(np.abs(got - ref)))
    assert err <= b, f"{what}: max err {err:.3e} > bound {b:.3e}"
    return err


@pytest.mark.parametrize("shift", [100.0, 1000.0])
def test_translated_mixture_trajectory(shift):
    """Cube against an 8-Gaussian mixture (the 70000-point workload's shapes, 3000
    points), eps = 0.01, 15 iterations, both clouds moved by (shift, shift, shift)."""
    p = translate(make_case(3000, 2800, 3, dist="mixture", seed=31, eps=0.01, iters=15), shift)
    X, Y, a, b = dev(p)
    ws = sk.alloc_workspace(X, Y)
    f, g = sk.solve(X, Y, a, b, 0.01, p.iters, ws=ws)
    flags = sk.range_flags(X, Y, ws)
    torch.cuda.synchronize()
    rf, rg = oracle.solve(p.X[0], p.Y[0], p.a[0], p.b[0], 0.01, p.iters)
    check(f[0].cpu().numpy(), rf, bound(p, 0.01, rf), f"f, shift {shift}")
    check(g[0].cpu().numpy(), rg, bound(p, 0.01, rg), f"g, shift {shift}")
    assert flags == 0, flags


def _rows(n, k, seed):
    rng = np.random.default_rng(seed)
    return np.sort(np.concatenate([rng.choice(n, size=k, replace=False), [0, n - 1]]))


@pytest.mark.parametrize("shift", [100.0, 1000.0])
def test_translated_full_size_half_steps(shift):
    """The 70000-point workload itself, moved by (shift, shift, shift): one half-step
    each way from seeded potentials at eps = 0.01, on sampled rows."""
    p = translate(make_config(3), shift)
    X, Y, a, b = dev(p)
    ws = sk.alloc_workspace(X, Y)
    sk.init_norms(X, Y, a, b, ws)
    g = random_potential((1, p.m), 3, 0.1)
    f_in = random_potential((1, p.n), 4, 0.1)
    f = sk.half_step_f(X, Y, ws, torch.from_numpy(g).cuda(), 0.01)
    gg = sk.half_step_g(X, Y, ws, torch.from_numpy(f_in).cuda(), 0.01)
    flags = sk.range_flags(X, Y, ws)
    torch.cuda.synchronize()
    rf_i, rg_i = _rows(p.n, 200, 5), _rows(p.m, 200, 6)
    ref_f = oracle.half_step_f(p.X[0], p.Y[0], p.b[0], g[0], 0.01, rows=rf_i)
    ref_g = oracle.half_step_g(p.X[0], p.Y[0], p.a[0], f_in[0], 0.01, rows=rg_i)
    check(f[0].cpu().numpy()[rf_i], ref_f, bound(p, 0.01, ref_f), f"f half-step, shift {shift}")
    check(gg[0].cpu().numpy()[rg_i], ref_g, bound(p, 0.01, ref_g), f"g half-step, shift {shift}")
    assert flags == 0, flags


def test_translated_bf16_is_centred_exactly():
    """bf16 clouds far from the origin: x - c is a bf16 value, so the centred bf16
    operands are exact and the bf16 bound holds (without centring the fp32
    accumulation of scores near |t|^2 would lose it)."""
    p = translate(make_case(700, 600, 64, seed=33, dtype="bf16", scale=1.0, eps=0.05, iters=10), 100.0)
    X, Y, a, b = dev(p)
    ws = sk.alloc_workspace(X, Y)
    f, g = sk.solve(X, Y, a, b, 0.05, p.iters, ws=ws)
    torch.cuda.synchronize()
    rf, rg = oracle.solve(p.X[0], p.Y[0], p.a[0], p.b[0], 0.05, p.iters)
    check(f[0].cpu().numpy(), rf, bound(p, 0.05, rf), "bf16 f")
    check(g[0].cpu().numpy(), rg, bound(p, 0.05, rg), "bf16 g")
    assert sk.range_flags(X, Y, ws) == 0


def test_translated_transport_returns_given_coordinates():
    """Barycentric projections come back in the given (uncentred) coordinates."""
    p = translate(make_case(500, 400, 3, dist="mixture", seed=34, eps=0.05), 250.0)
    X, Y, a, b = dev(p)
    rf, rg = oracle.solve(p.X[0], p.Y[0], p.a[0], p.b[0], 0.05, 5)
    f = torch.from_numpy(rf.astype(np.float32))[None].cuda()
    g = torch.from_numpy(rg.astype(np.float32))[None].cuda()
    ws = sk.alloc_workspace(X, Y, transport=True)
    sk.init_norms(X, Y, a, b, ws)
    bx, gx = sk.barycentric_x(X, Y, ws, f, g, 0.05)
    torch.cuda.synchronize()
    fr = rf.astype(np.float32).astype(np.float64)
    gr = rg.astype(np.float32).astype(np.float64)
    ref_b, ref_gr, _ = oracle.transport_x(p.X[0], p.Y[0], p.a[0], p.b[0], fr, gr, 0.05)
    spread = float(np.max(p.Y[0]) - np.min(p.Y[0]))
    check(bx[0].cpu().numpy(), ref_b, 2e-5 * max(spread, 1.0) + 4e-5, "bary")
    assert np.all(np.isfinite(gx.cpu().numpy()))


def test_translated_hvp_matches_dense_oracle():
    """The HVP at translated clouds (every coordinate the HVP reads is centred)."""
    p = translate(make_case(60, 50, 2, seed=35, eps=0.3, scale=0.7), 40.0)
    X, Y, a, b = dev(p)
    rf, rg = oracle.solve(p.X[0], p.Y[0], p.a[0], p.b[0], 0.3, 300)
    f = torch.from_numpy(rf.astype(np.float32))[None].cuda()
    g = torch.from_numpy(rg.astype(np.float32))[None].cuda()
    V = np.random.default_rng(3).standard_normal((1, 60, 2)).astype(np.float32)
    ws = sk.alloc_workspace(X, Y, hvp=True)
    sk.init_norms(X, Y, a, b, ws)
    hv = sk.hvp_x(X, Y, ws, f, g, 0.3, torch.from_numpy(V).cuda(), cg_iters=200, cg_tol=1e-10)
    torch.cuda.synchronize()
    ref = oracle.hvp_x(p.X[0], p.Y[0], p.a[0], p.b[0], rf.astype(np.float32), rg.astype(np.float32), 0.3, V[0])
    err = float(np.max(np.abs(hv[0].cpu().numpy() - ref)))
    assert err <= 5e-4 * float(np.max(np.abs(ref))), err


def test_scores_beyond_the_range_set_the_flag():
    """Spread 300 at eps = 1e-3: base-2 scores near 1e9, far past 2^22.  The kernels
    must report it (the potentials are then not trusted); a normal problem on the
    same workspace afterwards clears it at init."""
    p = make_case(300, 200, 3, seed=36, dist="cube", scale=300.0)
    X, Y, a, b = dev(p)
    ws = sk.alloc_workspace(X, Y)
    sk.solve(X, Y, a, b, 1e-3, 2, ws=ws)
    flags = sk.range_flags(X, Y, ws)
    assert flags & sk.SK_FLAG_SCORE_RANGE, flags
    q = make_case(300, 200, 3, seed=37)
    Xq, Yq, aq, bq = dev(q)
    sk.solve(Xq, Yq, aq, bq, 0.1, 2, ws=ws)
    assert sk.range_flags(Xq, Yq, ws) == 0
