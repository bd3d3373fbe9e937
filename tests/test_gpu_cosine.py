"""GPU parity of the cosine cost (page "FlashSinkhorn: Trasporto Ottimo Entropico Consapevole delle
I/O su GPU", section "Significato e Affermazioni": cosine distance after normalisation) through the
C ABI.

The oracle normalises the clouds in fp64 and runs its squared-Euclidean
routines on them; the raw-point gradient applies the chain rule through the
normalisation.  Bounds are those of the fp32 path (the cosine cost always runs
on the split fp32 layout): potentials 1e-3 eps + 1e-5 max|ref|; transport as in
the squared-Euclidean transport tests, with V the normalised other cloud.
"""

import numpy as np
import pytest
import torch

import oracle
from log_domain_sinkhorn_half_amd import binding as sk
from log_domain_sinkhorn_half_amd.inputs import make_case, random_potential

pytestmark = pytest.mark.gpu
COS = sk.SK_COSINE


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


def pot_tol(eps, ref):
    return 1e-3 * eps + 1e-5 * float(np.max(np.abs(ref)))


CASES = [(300, 200, 3, "fp32"), (129, 257, 16, "fp32"), (200, 150, 64, "fp32"), (96, 130, 88, "fp32"),
         (150, 170, 32, "bf16"), (77, 90, 64, "bf16")]


@pytest.mark.parametrize("n,m,d,dtype", CASES)
def test_cosine_half_steps_and_solve(n, m, d, dtype):
    p = make_case(n, m, d, seed=11 * n + d, weights="softmax", dtype=dtype, shift=0.3)
    X, Y, a, b = dev(p)
    Xh, Yh = oracle.normalize(p.X[0]), oracle.normalize(p.Y[0])
    ws = sk.alloc_workspace(X, Y, cost=COS)
    sk.init_norms(X, Y, a, b, ws, cost=COS)
    for eps in (0.5, 0.02):
        g = random_potential((1, m), d, 0.3)
        f_in = random_potential((1, n), d + 1, 0.3)
        f = sk.half_step_f(X, Y, ws, torch.from_numpy(g).cuda(), eps, cost=COS).cpu().numpy()
        gg = sk.half_step_g(X, Y, ws, torch.from_numpy(f_in).cuda(), eps, cost=COS).cpu().numpy()
        ref_f = oracle.half_step_f(Xh, Yh, p.b[0], g[0], eps)
        ref_g = oracle.half_step_g(Xh, Yh, p.a[0], f_in[0], eps)
        assert np.max(np.abs(f[0] - ref_f)) <= pot_tol(eps, ref_f)
        assert np.max(np.abs(gg[0] - ref_g)) <= pot_tol(eps, ref_g)
    eps = 0.05
    fs, gs = sk.solve(X, Y, a, b, eps, 10, cost=COS)
    rf, rg = oracle.solve(Xh, Yh, p.a[0], p.b[0], eps, 10)
    assert np.max(np.abs(fs.cpu().numpy()[0] - rf)) <= pot_tol(eps, rf)
    assert np.max(np.abs(gs.cpu().numpy()[0] - rg)) <= pot_tol(eps, rg)


@pytest.mark.parametrize("n,m,d,dtype", [(300, 200, 3, "fp32"), (200, 150, 64, "fp32"), (150, 170, 32, "bf16")])
def test_cosine_transport(n, m, d, dtype):
    p = make_case(n, m, d, seed=13 * n + d, weights="softmax", dtype=dtype, shift=0.3)
    p.X[0, 3] = 0.0  # a zero point: normalises to zero, zero raw gradient
    if dtype == "bf16":
        p.X_bits[0, 3] = 0
    X, Y, a, b = dev(p)
    Xr, Yr = p.X[0].astype(np.float64), p.Y[0].astype(np.float64)
    Xh, Yh = oracle.normalize(Xr), oracle.normalize(Yr)
    eps = 0.05
    f, g = oracle.solve(Xh, Yh, p.a[0], p.b[0], eps, 3)
    f, g = f.astype(np.float32), g.astype(np.float32)
    ws = sk.alloc_workspace(X, Y, transport=True, cost=COS)
    sk.init_norms(X, Y, a, b, ws, cost=COS)
    ft, gt = torch.from_numpy(f[None]).cuda(), torch.from_numpy(g[None]).cuda()
    bx, gx = sk.barycentric_x(X, Y, ws, ft, gt, eps, cost=COS)
    by, gy = sk.barycentric_y(X, Y, ws, ft, gt, eps, cost=COS)
    bx, gx, by, gy = (t.cpu().numpy()[0] for t in (bx, gx, by, gy))
    for side, bary, grad, P, Ph, V in (("x", bx, gx, Xr, Xh, Yh), ("y", by, gy, Yr, Yh, Xh)):
        if side == "x":
            rb, rgh, rm = oracle.transport_x(Xh, Yh, p.a[0], p.b[0], f, g, eps)
            T = oracle.half_step_f(Xh, Yh, p.b[0], g, eps)
        else:
            rb, rgh, rm = oracle.transport_y(Xh, Yh, p.a[0], p.b[0], f, g, eps)
            T = oracle.half_step_g(Xh, Yh, p.a[0], f, eps)
        rg = oracle.cosine_grad(P, rgh)
        tb = 2e-5 * float(np.max(np.abs(V)))
        assert np.max(np.abs(bary - rb)) <= tb, side
        dm = np.expm1((1e-3 * eps + 1e-5 * float(np.max(np.abs(T)))) / eps)
        nrm = np.sqrt((P * P).sum(1))
        inv = np.divide(1.0, nrm, out=np.zeros_like(nrm), where=nrm > 0)
        # the chain rule is a projection (norm <= 1) scaled by 1/|p|: a row's error is
        # at most the 2-norm of its normalised-point bound over |p|
        tgh = 2.0 * rm[:, None] * (tb * (1.0 + dm) + np.abs(Ph - rb) * dm)
        tg = np.sqrt((tgh ** 2).sum(1)) * inv
        assert np.all(np.abs(grad - rg) <= tg[:, None]), side
    assert np.all(gx[3] == 0.0)
    np.testing.assert_allclose((gx * Xr).sum(1), 0.0, atol=1e-5 * np.abs(gx * Xr).sum())


def test_cosine_scale_invariance_on_gpu():
    p = make_case(200, 180, 8, seed=5, weights="softmax")
    X, Y, a, b = dev(p)
    s = torch.from_numpy(np.random.default_rng(1).uniform(0.5, 4.0, (1, 200, 1)).astype(np.float32)).cuda()
    f1, g1 = sk.solve(X, Y, a, b, 0.05, 10, cost=COS)
    f2, g2 = sk.solve((X * s).contiguous(), Y, a, b, 0.05, 10, cost=COS)
    ref = f1.cpu().numpy()
    assert np.max(np.abs(f1.cpu().numpy() - f2.cpu().numpy())) <= pot_tol(0.05, ref)
