"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Acceptance bound (per half-step output and per trajectory):
  fp32 inputs: max|pot_gpu - pot_ref| <= 1e-3*eps + 1e-5*max|pot_ref|
  bf16 inputs: max|pot_gpu - pot_ref| <= 2e-2*eps   (eps = the last eps used)
Both sides read identical seeded inputs (bf16 problems: the exact bf16 values).
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
    sk.load_library()  # raises loudly if the HIP library is missing


def dev(p):
    if p.dtype == "bf16":
        X = torch.from_numpy(p.X_bits.view(np.int16)).cuda().view(torch.bfloat16)
        Y = torch.from_numpy(p.Y_bits.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        X = torch.from_numpy(p.X).cuda()
        Y = torch.from_numpy(p.Y).cuda()
    return X, Y, torch.from_numpy(p.a).cuda(), torch.from_numpy(p.b).cuda()


def tol(p, eps, ref):
    if p.dtype == "bf16":
        return 2e-2 * eps
    return 1e-3 * eps + 1e-5 * float(np.max(np.abs(ref)))


def check(gpu, ref, bound, what):
    gpu = np.asarray(gpu, np.float64)
    err = np.max(np.abs(gpu - ref))
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    assert err <= bound, f"{what}: max err {err:.3e} > bound {bound:.3e}"
    return err


def half_steps(p, eps, seed, rows=None, scale=0.3):
    """GPU f and g half-steps from seeded potentials vs oracle (optionally on sampled rows)."""
    X, Y, a, b = dev(p)
    ws = sk.alloc_workspace(X, Y)
    sk.init_norms(X, Y, a, b, ws)
    g = random_potential((p.batch, p.m), seed, scale)
    f_in = random_potential((p.batch, p.n), seed + 1, scale)
    f = sk.half_step_f(X, Y, ws, torch.from_numpy(g).cuda(), eps)
    gg = sk.half_step_g(X, Y, ws, torch.from_numpy(f_in).cuda(), eps)
    torch.cuda.synchronize()
    f, gg = f.cpu().numpy(), gg.cpu().numpy()
    for k in range(p.batch):
        rf = None if rows is None else rows[0]
        rg = None if rows is None else rows[1]
        ref_f = oracle.half_step_f(p.X[k], p.Y[k], p.b[k], g[k], eps, rows=rf)
        ref_g = oracle.half_step_g(p.X[k], p.Y[k], p.a[k], f_in[k], eps, rows=rg)
        got_f = f[k] if rf is None else f[k][rf]
        got_g = gg[k] if rg is None else gg[k][rg]
        check(got_f, ref_f, tol(p, eps, ref_f), f"f half-step problem {k}")
        check(got_g, ref_g, tol(p, eps, ref_g), f"g half-step problem {k}")


# ---------------------------------------------------------------------------
# half-steps on ragged shapes spanning several tiles, every supported K width
# ---------------------------------------------------------------------------
SHAPES = [
    (1, 1, 3), (1, 7, 3), (7, 1, 2), (63, 65, 3), (65, 63, 4), (1000, 777, 3), (777, 1000, 1),
    (300, 513, 5), (513, 300, 9), (257, 1029, 17), (1030, 255, 32), (129, 700, 64), (700, 129, 88),
    (200, 333, 80), (150, 140, 4), (140, 150, 12),
    # d <= 3 past 2^21 scores with fewer than 16384 keys: 128-key chunks and key splits
    # (the smaller d <= 3 shapes above take one launch without splits)
    (3001, 1500, 3), (1500, 3001, 2),
]


@pytest.mark.parametrize("n,m,d", SHAPES)
def test_half_steps_fp32_ragged(n, m, d):
    p = make_case(n, m, d, seed=n + m + d, weights="softmax", scale=1.0 / np.sqrt(d))
    for eps in (0.5, 0.05):
        half_steps(p, eps, seed=d)


@pytest.mark.parametrize("n,m,d", [(1, 5, 8), (63, 65, 8), (1000, 777, 32), (300, 1100, 64),
                                   (333, 200, 128), (129, 515, 96), (77, 90, 40)])
def test_half_steps_bf16_ragged(n, m, d):
    p = make_case(n, m, d, seed=7 * n + m, weights="softmax", dtype="bf16", scale=1.0 / np.sqrt(d))
    for eps in (1.0, 0.1, 0.01):
        half_steps(p, eps, seed=d)


@pytest.mark.parametrize("n,m,d", [(200, 150, 200), (129, 260, 256), (100, 90, 300), (70, 130, 512),
                                   (64, 65, 777), (50, 60, 1024)])
def test_half_steps_bf16_wide(n, m, d):
    """bf16 operands past 256 slots take 16x16 tiles with one query tile per wave."""
    p = make_case(n, m, d, seed=3 * n + d, weights="softmax", dtype="bf16", scale=1.0 / np.sqrt(d))
    for eps in (1.0, 0.05):
        half_steps(p, eps, seed=d)


def test_solve_bf16_wide_trajectory():
    p = make_case(150, 170, 512, seed=12, weights="softmax", dtype="bf16", scale=1.0 / np.sqrt(512), iters=20)
    X, Y, a, b = dev(p)
    f, g = sk.solve(X, Y, a, b, 0.05, p.iters)
    rf, rg = oracle.solve(p.X[0], p.Y[0], p.a[0], p.b[0], 0.05, p.iters)
    check(f.cpu().numpy()[0], rf, tol(p, 0.05, rf), "bf16 d=512 f")
    check(g.cpu().numpy()[0], rg, tol(p, 0.05, rg), "bf16 d=512 g")


def test_half_steps_batched_small():
    p = make_case(70, 90, 6, batch=5, seed=3, weights="softmax")
    half_steps(p, 0.2, seed=3)


# ---------------------------------------------------------------------------
# full trajectories
# ---------------------------------------------------------------------------
def gpu_solve(p, iters=None):
    X, Y, a, b = dev(p)
    it = p.iters if iters is None else iters
    eps = p.eps.tolist() if p.eps.size > 1 else float(p.eps[0])
    f, g = sk.solve(X, Y, a, b, eps, it)
    torch.cuda.synchronize()
    return f.cpu().numpy(), g.cpu().numpy()


@pytest.mark.parametrize("n,m,d,eps,iters", [(1000, 777, 3, 0.05, 20), (513, 1000, 16, 0.1, 15),
                                             (600, 450, 64, 0.2, 10)])
def test_trajectory_small(n, m, d, eps, iters):
    p = make_case(n, m, d, eps=eps, iters=iters, seed=n, weights="softmax", scale=1.0 / np.sqrt(d))
    f, g = gpu_solve(p)
    rf, rg = oracle.solve(p.X[0], p.Y[0], p.a[0], p.b[0], eps, iters)
    check(f[0], rf, tol(p, eps, rf), "f")
    check(g[0], rg, tol(p, eps, rg), "g")


def test_config1_full_trajectory():
    p = make_config(1)
    f, g = gpu_solve(p)
    rf, rg = oracle.solve(p.X, p.Y, p.a, p.b, float(p.eps[0]), p.iters)
    e = float(p.eps[0])
    check(f, rf, tol(p, e, rf), "C1 f")
    check(g, rg, tol(p, e, rg), "C1 g")


def test_config5_batched_trajectory_sampled_problems():
    p = make_config(5)
    f, g = gpu_solve(p)
    e = float(p.eps[0])
    for k in (0, 37, 63):
        rf, rg = oracle.solve(p.X[k], p.Y[k], p.a[k], p.b[k], e, p.iters)
        check(f[k], rf, tol(p, e, rf), f"C5 f problem {k}")
        check(g[k], rg, tol(p, e, rg), f"C5 g problem {k}")


def test_config5_half_steps_all_rows_sampled_problems():
    # Launch shape of the batched workload (2 key splits, 64 chunks per split): the
    # running offset must jump by more than 126 while partial sums are ~2^100+.
    p = make_config(5)
    X, Y, a, b = dev(p)
    ws = sk.alloc_workspace(X, Y)
    sk.init_norms(X, Y, a, b, ws)
    e = float(p.eps[0])
    for seed, scale in ((None, 0.0), (5, 3.0)):
        g = np.zeros((p.batch, p.m), np.float32) if seed is None else random_potential((p.batch, p.m), seed, scale)
        f = sk.half_step_f(X, Y, ws, torch.from_numpy(g).cuda(), e)
        torch.cuda.synchronize()
        f = f.cpu().numpy()
        for k in (0, 21, 63):
            ref = oracle.half_step_f(p.X[k], p.Y[k], p.b[k], g[k], e)
            check(f[k], ref, tol(p, e, ref), f"C5 f half-step problem {k}")


# ---------------------------------------------------------------------------
# full-size workloads: one half-step each way on sampled rows
# ---------------------------------------------------------------------------
def _rows(n, k, seed):
    rng = np.random.default_rng(seed)
    r = rng.choice(n, size=min(k, n), replace=False)
    return np.sort(np.concatenate([r, [0, n - 1]]))


@pytest.mark.parametrize("cfg", [2, 3])
def test_full_size_half_steps_sampled(cfg):
    p = make_config(cfg)
    eps = float(p.eps[-1])
    half_steps(p, eps, seed=cfg, rows=(_rows(p.n, 256, cfg), _rows(p.m, 256, cfg + 1)), scale=0.1)


@pytest.mark.parametrize("eps", [1.0, 0.1, 0.01])
def test_full_size_bf16_half_steps_sampled(eps):
    p = make_config(4)
    half_steps(p, eps, seed=4, rows=(_rows(p.n, 128, 4), _rows(p.m, 128, 5)), scale=0.1)


# ---------------------------------------------------------------------------
# properties: determinism, symmetry, resume, batching, marginals
# ---------------------------------------------------------------------------
def test_bitwise_determinism_and_role_swap():
    p = make_case(900, 1300, 3, seed=5, weights="softmax")
    X, Y, a, b = dev(p)
    ws = sk.alloc_workspace(X, Y)
    sk.init_norms(X, Y, a, b, ws)
    g = torch.from_numpy(random_potential((1, p.m), 5)).cuda()
    f1 = sk.half_step_f(X, Y, ws, g, 0.07).clone()
    f2 = sk.half_step_f(X, Y, ws, g, 0.07).clone()
    # g half-step of the swapped problem (Y as sources) == f half-step of the original
    ws2 = sk.alloc_workspace(Y, X)
    sk.init_norms(Y, X, b, a, ws2)
    f3 = sk.half_step_g(Y, X, ws2, g, 0.07)
    torch.cuda.synchronize()
    assert torch.equal(f1, f2)
    assert torch.equal(f1, f3)


def test_resume_equals_uninterrupted():
    p = make_case(800, 700, 3, seed=6, weights="softmax")
    X, Y, a, b = dev(p)
    f, g = sk.solve(X, Y, a, b, 0.05, 30)
    f2, g2 = sk.solve(X, Y, a, b, 0.05, 18)
    f2, g2 = sk.solve(X, Y, a, b, 0.05, 12, f=f2, g=g2)
    torch.cuda.synchronize()
    assert torch.equal(f, f2) and torch.equal(g, g2)


def test_batched_equals_single_problems():
    p = make_case(500, 600, 8, batch=6, seed=7)
    X, Y, a, b = dev(p)
    f, g = sk.solve(X, Y, a, b, 0.1, 8)
    for k in range(6):
        fk, gk = sk.solve(X[k:k + 1].contiguous(), Y[k:k + 1].contiguous(), a[k:k + 1].contiguous(),
                          b[k:k + 1].contiguous(), 0.1, 8)
        torch.cuda.synchronize()
        ref = oracle.solve(p.X[k], p.Y[k], p.a[k], p.b[k], 0.1, 8)
        check(fk[0].cpu().numpy(), f[k].cpu().numpy().astype(np.float64), tol(p, 0.1, ref[0]), "batched f")
        check(gk[0].cpu().numpy(), g[k].cpu().numpy().astype(np.float64), tol(p, 0.1, ref[1]), "batched g")


def test_annealed_schedule_matches_oracle():
    p = make_case(700, 500, 3, seed=8, weights="softmax")
    sched = (1.0 * (0.02 / 1.0) ** (np.arange(12) / 11)).astype(np.float32)
    X, Y, a, b = dev(p)
    f, g = sk.solve(X, Y, a, b, sched.tolist(), 12)
    torch.cuda.synchronize()
    rf, rg = oracle.solve(p.X[0], p.Y[0], p.a[0], p.b[0], sched.astype(np.float64), 12)
    check(f[0].cpu().numpy(), rf, tol(p, float(sched[-1]), rf), "annealed f")
    check(g[0].cpu().numpy(), rg, tol(p, float(sched[-1]), rg), "annealed g")


@pytest.mark.parametrize("d", [3, 32])
def test_key_operand_reuse_across_eps_and_clouds(d):
    """The fp32 key operands keep their coordinate parts between half-steps at one
    eps and rebuild them when eps changes, after a plan product at another eps, and
    after init_norms with new clouds on the same workspace: every step here is
    checked against the oracle."""
    p = make_case(300, 200, d, seed=12 + d, weights="softmax", scale=1.0 / np.sqrt(d))
    q = make_case(300, 200, d, seed=40 + d, weights="softmax", scale=1.0 / np.sqrt(d))
    X, Y, a, b = dev(p)
    ws = sk.alloc_workspace(X, Y, transport=True)
    sk.init_norms(X, Y, a, b, ws)
    g1 = random_potential((1, 200), 21, 0.3)
    g2 = random_potential((1, 200), 22, 0.3)
    f1 = random_potential((1, 300), 23, 0.3)

    def step_f(Xc, Yc, pc, g, eps, what):
        out = sk.half_step_f(Xc, Yc, ws, torch.from_numpy(g).cuda(), eps)
        torch.cuda.synchronize()
        ref = oracle.half_step_f(pc.X[0], pc.Y[0], pc.b[0], g[0], eps)
        check(out[0].cpu().numpy(), ref, tol(pc, eps, ref), what)

    step_f(X, Y, p, g1, 0.1, "first build")
    step_f(X, Y, p, g2, 0.1, "same eps, new potential")
    gg = sk.half_step_g(X, Y, ws, torch.from_numpy(f1).cuda(), 0.1)  # the other side's operand
    torch.cuda.synchronize()
    ref = oracle.half_step_g(p.X[0], p.Y[0], p.a[0], f1[0], 0.1)
    check(gg[0].cpu().numpy(), ref, tol(p, 0.1, ref), "g side")
    step_f(X, Y, p, g1, 0.1, "f side again")
    step_f(X, Y, p, g1, 0.03, "new eps")
    V = np.random.default_rng(3).standard_normal((1, 200)).astype(np.float32)
    sk.apply_plan_x(X, Y, ws, torch.from_numpy(f1).cuda(), torch.from_numpy(g2).cuda(), 0.5,
                    torch.from_numpy(V).cuda())
    step_f(X, Y, p, g2, 0.03, "after a plan product at another eps")
    Xq, Yq, aq, bq = dev(q)
    sk.init_norms(Xq, Yq, aq, bq, ws)
    step_f(Xq, Yq, q, g2, 0.03, "new clouds, same eps")


def test_marginal_error_matches_oracle_plan():
    p = make_case(400, 300, 3, seed=9, weights="softmax")
    eps = 0.1
    X, Y, a, b = dev(p)
    ws = sk.alloc_workspace(X, Y)
    f, g = sk.solve(X, Y, a, b, eps, 5, ws=ws)
    err = sk.marginal_error(X, Y, ws, f, g, eps)
    torch.cuda.synchronize()
    fn, gn = f[0].cpu().numpy().astype(np.float64), g[0].cpu().numpy().astype(np.float64)
    ra, cb = oracle.marginal_error(p.X[0], p.Y[0], p.a[0], p.b[0], fn, gn, eps)
    e = err.cpu().numpy()[0]
    # after a g half-step the columns match b up to fp32 rounding; rows carry the real error
    assert abs(e[0] - ra) <= 1e-3 * ra + 2e-5, (e, ra)
    assert e[1] <= 2e-5 and cb <= 1e-5, (e, cb)


def test_zero_weight_point_is_removed():
    p = make_case(300, 200, 3, seed=10, weights="softmax")
    b = p.b.copy()
    b[0, 17] = 0.0
    X, Y, a, _ = dev(p)
    bt = torch.from_numpy(b).cuda()
    ws = sk.alloc_workspace(X, Y)
    sk.init_norms(X, Y, a, bt, ws)
    g = random_potential((1, 200), 10)
    f = sk.half_step_f(X, Y, ws, torch.from_numpy(g).cuda(), 0.05)
    torch.cuda.synchronize()
    ref = oracle.half_step_f(p.X[0], p.Y[0], b[0], g[0], 0.05)
    check(f[0].cpu().numpy(), ref, tol(p, 0.05, ref), "zero-weight f")


def test_large_dynamic_range_forces_offset_moves():
    # scores spanning thousands of base-2 units: the lazy offset must move many times
    p = make_case(333, 2000, 2, seed=11, weights="softmax", dist="cube", scale=8.0)
    half_steps(p, 0.01, seed=11, scale=5.0)


# ---------------------------------------------------------------------------
# full-size trajectories at sampled indices (fixtures written by
# tests/golden/make_golden.py from the oracle alone)
# ---------------------------------------------------------------------------
def _golden(cfg):
    import hashlib
    import json
    import os

    path = os.path.join(os.path.dirname(__file__), "golden", f"trajectory_config{cfg}.json")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated (python tests/golden/make_golden.py {cfg})")
    gold = json.load(open(path))
    p = make_config(cfg)
    h = hashlib.sha256()
    for arr in (p.X, p.Y, p.a, p.b, p.eps):
        h.update(np.ascontiguousarray(arr).tobytes())
    assert h.hexdigest()[:16] == gold["inputs_sha256_16"], "inputs changed since the fixture was written"
    return p, gold


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_full_trajectory_against_golden_samples(cfg):
    p, gold = _golden(cfg)
    f, g = gpu_solve(p)
    e = float(p.eps[-1])
    rf = np.array(gold["f"])
    rg = np.array(gold["g"])
    if p.dtype == "bf16":
        bf = bg = 2e-2 * e  # the final eps of the annealing schedule
    else:
        bf = 1e-3 * e + 1e-5 * gold["f_absmax"]
        bg = 1e-3 * e + 1e-5 * gold["g_absmax"]
    # indices run over the problem-major flattened potentials (one problem: the rows)
    check(f.reshape(-1)[gold["f_index"]], rf, bf, f"C{cfg} f trajectory")
    check(g.reshape(-1)[gold["g_index"]], rg, bg, f"C{cfg} g trajectory")


def test_config4_every_annealed_iteration_against_golden():
    """The 65536 x 32768 d = 128 bf16 workload, eps annealed 1.0 -> 0.01 over 100
    iterations: after every iteration k, f_k and g_k at 64 sampled indices per side
    against the oracle's trajectory (fixture written by make_golden.py --per-iter),
    so each of the 200 half-steps is checked, not only the last.  The GPU runs the
    schedule one solve call per iteration (resuming from its own g), which is the
    same sequence of kernels and values as one call with the whole schedule."""
    p, gold = _golden(4)
    if "per_iter_f" not in gold:
        pytest.skip("fixture has no per-iteration samples")
    X, Y, a, b = dev(p)
    ws = sk.alloc_workspace(X, Y)
    f = torch.zeros((1, p.n), dtype=torch.float32, device="cuda")
    g = torch.zeros((1, p.m), dtype=torch.float32, device="cuda")
    fi, gi = gold["per_iter_f_index"], gold["per_iter_g_index"]
    bound = 2e-2 * float(p.eps[-1])
    worst = 0.0
    for k in range(p.iters):
        sk.solve(X, Y, a, b, float(p.eps[k]), 1, f=f, g=g, ws=ws)
        torch.cuda.synchronize()
        fk = f[0].cpu().numpy()[fi]
        gk = g[0].cpu().numpy()[gi]
        worst = max(worst, check(fk, np.array(gold["per_iter_f"][k]), bound, f"C4 f after iteration {k}"),
                    check(gk, np.array(gold["per_iter_g"][k]), bound, f"C4 g after iteration {k}"))
    print(f"C4 per-iteration worst error {worst:.3e} (bound {bound:.1e})")
    # the one-call annealed solve agrees with the iteration-by-iteration one
    f2, g2 = gpu_solve(p)
    assert np.array_equal(f2[0], f[0].cpu().numpy()) and np.array_equal(g2[0], g[0].cpu().numpy())
