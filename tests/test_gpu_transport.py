"""GPU parity of the transport application (barycentric projection and gradient)
through the C ABI against the fp64 oracle (page "FlashSinkhorn: Trasporto Ottimo Entropico
Consapevole delle I/O su GPU", section "Metodologia", part "3. Differenziazione e Ottimizzazione del
Secondo Ordine").

Acceptance bounds, derived from the arithmetic of the two passes:
  bary: fp32 inputs |d bary| <= 2e-5 * max|V|, bf16 inputs <= 5e-4 * max|V| for d <= 128,
        V = the other cloud; past d = 128 the bf16 bound grows with the score's number
        of fp32 roundings, d/8 + 2 (measured at eps = 0.01: 4.7e-4 at d = 200 and
        5.8e-4 at d = 256 against bounds of 7.5e-4 and 9.4e-4).  The weights carry the
        score rounding of the half-step kernel (about 1e-6 relative for fp32 operands, 2.5e-5 for bf16
        operands at lambda = log2(e)/0.01) and a 2^-17 two-part bf16 split (fp32
        inputs); a convex combination moves by at most that relative error times the
        spread of V.  bf16 inputs take fp16 weights (rounded to nearest, 2^-11
        relative, the sums formed from the same rounded values) against exact fp16
        values: each normalised weight moves by at most 2^-10 relative, so the average
        moves by at most 2^-10 times its weighted deviation, which is at most half
        the range of V's coordinate (Popoviciu); that term is added.
  grad: 2 r_i (tol_bary + |x_i - bary_i| * tol_T / eps), where r_i is the row mass
        and tol_T the half-step bound (1e-3 eps + 1e-5 max|T| for fp32, 2e-2 eps for
        bf16): the mass comes from the row log-sum-exp of the half-step.
Potentials come from the oracle (a few oracle iterations, or an oracle half-step
on sampled rows) or from the seeded generator, never from the HIP path.
"""

import numpy as np
import pytest
import torch

import oracle
from log_domain_sinkhorn_half_amd import binding as sk
from log_domain_sinkhorn_half_amd.inputs import make_case, make_config, random_potential

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


def bounds(p, eps, V, P, bary_ref, mass_ref, T_ref):
    rel = 5e-4 if p.dtype == "bf16" else 2e-5
    d = V.shape[1]
    if p.dtype == "bf16" and d > 128:
        # the score's rounding error grows with its d/8 + 2 fp32 roundings (groups of
        # 8 exact bf16 products, the bias, the base-2 scaling); 5e-4 holds up to d = 128
        rel *= (d / 8 + 2) / (128 / 8 + 2)
    tb = rel * float(np.max(np.abs(V)))
    if p.dtype == "bf16":
        # fp16 weights of the transport pass: 2^-10 of half the coordinate's range
        tb = tb + 2.0 ** -10 * 0.5 * (np.max(V, axis=0) - np.min(V, axis=0))[None, :]
    tT = 2e-2 * eps if p.dtype == "bf16" else 1e-3 * eps + 1e-5 * float(np.max(np.abs(T_ref)))
    dm = np.expm1(tT / eps)  # largest relative error of the row mass
    tg = 2.0 * mass_ref[:, None] * (tb * (1.0 + dm) + np.abs(P - bary_ref) * dm)
    return tb, tg


def compare(p, k, side, eps, bary, grad, f, g, rows=None):
    """Check problem k's GPU outputs (on `rows`, default all) against the oracle."""
    X, Y, a, b = (np.asarray(v[k], np.float64) for v in (p.X, p.Y, p.a, p.b))
    if side == "x":
        P, V, T_ref = X, Y, oracle.half_step_f(X, Y, b, g[k], eps, rows=rows)
        ref = oracle.transport_x(X, Y, a, b, f[k], g[k], eps, rows=rows)
    else:
        P, V, T_ref = Y, X, oracle.half_step_g(X, Y, a, f[k], eps, rows=rows)
        ref = oracle.transport_y(X, Y, a, b, f[k], g[k], eps, rows=rows)
    bary_ref, grad_ref, mass_ref = ref
    Psel = P if rows is None else P[rows]
    got_b = bary[k] if rows is None else bary[k][rows]
    tb, tg = bounds(p, eps, V, Psel, bary_ref, mass_ref, T_ref)
    assert np.all(np.isfinite(got_b)), f"{side} bary non-finite"
    err = np.abs(got_b - bary_ref)
    err_b = float(np.max(err))
    worst = float(np.max(err / np.broadcast_to(tb, err.shape)))
    print(f"bary_{side} {p.dtype} d={p.d} eps={eps}: max err {err_b:.2e}, worst err/bound {worst:.3f}")
    assert worst <= 1.0, f"bary_{side} problem {k}: max err {err_b:.3e}, worst err/bound {worst:.3f}"
    if grad is not None:
        got_g = grad[k] if rows is None else grad[k][rows]
        assert np.all(np.isfinite(got_g)), f"{side} grad non-finite"
        excess = np.abs(got_g - grad_ref) - tg
        assert np.all(excess <= 0), (f"grad_{side} problem {k}: worst err "
                                     f"{np.max(np.abs(got_g - grad_ref)):.3e}, worst excess {excess.max():.3e}")
    return err_b


def run_gpu(p, f, g, eps, with_grad=True):
    X, Y, a, b = dev(p)
    ws = sk.alloc_workspace(X, Y, transport=True)
    sk.init_norms(X, Y, a, b, ws)
    ft = torch.from_numpy(np.asarray(f, np.float32)).cuda()
    gt = torch.from_numpy(np.asarray(g, np.float32)).cuda()
    bx, gx = sk.barycentric_x(X, Y, ws, ft, gt, eps, with_grad=with_grad)
    by, gy = sk.barycentric_y(X, Y, ws, ft, gt, eps, with_grad=with_grad)
    torch.cuda.synchronize()
    cpu = lambda t: None if t is None else t.cpu().numpy()  # noqa: E731
    return cpu(bx), cpu(gx), cpu(by), cpu(gy)


def oracle_potentials(p, eps, iters=3):
    f, g = oracle.solve(p.X, p.Y, p.a, p.b, eps, iters)
    return f.astype(np.float32).astype(np.float64), g.astype(np.float32).astype(np.float64)


SHAPES_FP32 = [(1, 1, 3), (7, 1, 2), (1, 9, 3), (700, 129, 3), (200, 333, 1), (150, 140, 4),
               (64, 1000, 16), (301, 77, 33), (96, 130, 64), (40, 50, 88), (513, 300, 9)]


@pytest.mark.parametrize("n,m,d", SHAPES_FP32)
def test_transport_fp32_ragged(n, m, d):
    p = make_case(n, m, d, seed=3 * n + m + d, weights="softmax", scale=1.0 / np.sqrt(d))
    for eps in (0.5, 0.05):
        f, g = oracle_potentials(p, eps)
        bx, gx, by, gy = run_gpu(p, f, g, eps)
        compare(p, 0, "x", eps, bx, gx, f, g)
        compare(p, 0, "y", eps, by, gy, f, g)


@pytest.mark.parametrize("n,m,d", [(300, 200, 3), (129, 257, 64), (100, 90, 128), (63, 65, 8), (70, 90, 200),
                                   (60, 75, 256)])
def test_transport_bf16_ragged(n, m, d):
    p = make_case(n, m, d, seed=5 * n + m, weights="softmax", dtype="bf16", scale=1.0 / np.sqrt(d))
    for eps in (1.0, 0.1, 0.01):
        f, g = oracle_potentials(p, eps)
        bx, gx, by, gy = run_gpu(p, f, g, eps)
        compare(p, 0, "x", eps, bx, gx, f, g)
        compare(p, 0, "y", eps, by, gy, f, g)


def test_transport_batched_and_without_grad():
    p = make_case(70, 90, 6, batch=4, seed=9, weights="softmax")
    eps = 0.2
    f, g = oracle_potentials(p, eps)
    bx, gx, by, gy = run_gpu(p, f, g, eps)
    bx2, gx2, by2, gy2 = run_gpu(p, f, g, eps, with_grad=False)
    assert gx2 is None and gy2 is None
    np.testing.assert_array_equal(bx, bx2)  # same kernels, same order
    np.testing.assert_array_equal(by, by2)
    for k in range(p.batch):
        compare(p, k, "x", eps, bx, gx, f, g)
        compare(p, k, "y", eps, by, gy, f, g)


@pytest.mark.parametrize("shift", [0.0, 40.0])
def test_transport_bf16_batched_translated_zero_weights(shift):
    """bf16 inputs (fp16 weights and values in the transport pass): three problems of
    different spread, moved by `shift` in every coordinate (the library centres the
    clouds and scales their coordinates into fp16 per problem), with zero weights."""
    from log_domain_sinkhorn_half_amd.inputs import translate

    p = make_case(150, 170, 48, batch=3, seed=61, weights="softmax", dtype="bf16", scale=1.0 / np.sqrt(48))
    p.X[1] *= 4.0  # a wider problem next to narrow ones (rounded to bf16 again by translate)
    p.Y[1] *= 4.0
    p = translate(p, shift)
    p.a[0, 3] = 0.0
    p.b[2, 7] = 0.0
    for eps in (0.5, 0.02):
        f, g = oracle_potentials(p, eps)
        bx, gx, by, gy = run_gpu(p, f, g, eps)
        for k in range(p.batch):
            compare(p, k, "x", eps, bx, gx, f, g)
            compare(p, k, "y", eps, by, gy, f, g)
        assert np.all(gx[0, 3] == 0.0)  # a point of zero weight carries no mass


def test_transport_zero_weight_and_translation_balance():
    p = make_case(120, 150, 3, seed=21, weights="softmax")
    p.a[0, 5] = 0.0
    p.b[0, 17] = 0.0
    eps = 0.1
    f = random_potential((1, p.n), 31, 0.2).astype(np.float64)
    g = random_potential((1, p.m), 32, 0.2).astype(np.float64)
    bx, gx, by, gy = run_gpu(p, f, g, eps)
    compare(p, 0, "x", eps, bx, gx, f, g)
    compare(p, 0, "y", eps, by, gy, f, g)
    assert gx[0, 5].tolist() == [0.0, 0.0, 0.0]  # a point of zero weight carries no mass
    scale = np.abs(gx).sum() + np.abs(gy).sum()
    assert np.max(np.abs(gx[0].sum(0) + gy[0].sum(0))) <= 1e-4 * scale


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_transport_full_size_sampled(cfg):
    """Full-size workloads: GPU over all rows, oracle on sampled rows (and the last)."""
    p = make_config(cfg)
    eps = float(p.eps[-1])
    rng = np.random.default_rng(400 + cfg)
    k = rng.integers(0, p.batch)
    rx = np.unique(np.concatenate([rng.choice(p.n, size=min(48, p.n), replace=False), [p.n - 1]]))
    ry = np.unique(np.concatenate([rng.choice(p.m, size=min(48, p.m), replace=False), [p.m - 1]]))
    g = random_potential((p.batch, p.m), 40 + cfg, 0.1).astype(np.float64)
    f = random_potential((p.batch, p.n), 50 + cfg, 0.1).astype(np.float64)
    # on the checked rows the row's own potential is its exact update, so the row mass is the weight
    X, Y, a, b = (np.asarray(v[k], np.float64) for v in (p.X, p.Y, p.a, p.b))
    f_x = f.copy()
    f_x[k, rx] = oracle.half_step_f(X, Y, b, g[k], eps, rows=rx).astype(np.float32)
    g_y = g.copy()
    g_y[k, ry] = oracle.half_step_g(X, Y, a, f[k], eps, rows=ry).astype(np.float32)
    bx, gx, _, _ = run_gpu(p, f_x, g, eps)
    compare(p, k, "x", eps, bx, gx, f_x, g, rows=rx)
    _, _, by, gy = run_gpu(p, f, g_y, eps)
    compare(p, k, "y", eps, by, gy, f, g_y, rows=ry)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_transport_large_dynamic_range(dtype):
    """Scores spanning thousands of base-2 units: the transport pass's lazy row
    offsets must rise many times (and differ between key splits) without loss.
    Each side's own potential is the oracle's exact update, so row masses are the
    weights (a random one would put exp((f - lse)/eps) out of range)."""
    p = make_case(333, 2000, 2, seed=11, weights="softmax", dist="cube", scale=8.0, dtype=dtype)
    eps = 0.01
    X, Y, a, b = (np.asarray(v[0], np.float64) for v in (p.X, p.Y, p.a, p.b))
    g0 = random_potential((1, p.m), 62, 5.0).astype(np.float64)
    f = oracle.half_step_f(X, Y, b, g0[0], eps).astype(np.float32).astype(np.float64)[None, :]
    g1 = oracle.half_step_g(X, Y, a, f[0], eps).astype(np.float32).astype(np.float64)[None, :]
    bx, gx, _, _ = run_gpu(p, f, g0, eps)
    compare(p, 0, "x", eps, bx, gx, f, g0)
    _, _, by, gy = run_gpu(p, f, g1, eps)
    compare(p, 0, "y", eps, by, gy, f, g1)
    # keys sorted far to near from the first query: its offset rises block after block
    order = np.argsort(-((p.Y[0] - p.X[0][0]) ** 2).sum(1))
    q = make_case(333, 2000, 2, seed=11, weights="softmax", dist="cube", scale=8.0, dtype=dtype)
    q.Y[0] = p.Y[0][order]
    q.b[0] = p.b[0][order]
    if dtype == "bf16":
        q.Y_bits[0] = p.Y_bits[0][order]
    bx, gx, _, _ = run_gpu(q, f, g0[:, order], eps)
    compare(q, 0, "x", eps, bx, gx, f, g0[:, order])
