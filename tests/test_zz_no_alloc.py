"""The allocation-free solve (sinkhorn_solve_noalloc) through the C ABI.

It runs the solver on the library's built-in scratch array instead of a
caller's workspace.  Its output must equal sinkhorn_solve's on the same inputs
(the same kernels run in the same order, so the potentials agree bit for bit),
and both must meet the oracle bound.  Two calls in a row, the second on a
smaller problem, check that the array's leftover contents from the first call
do not leak into the second.  Host-side rejection (problems too large for the
array, NULL pointers) is checked without a GPU.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from log_domain_sinkhorn_half_amd import binding as sk
from log_domain_sinkhorn_half_amd.inputs import make_case


def _bound(eps, ref):
    return 1e-3 * eps + 1e-5 * float(np.max(np.abs(ref)))


def test_noalloc_rejects_on_the_host():
    lib = sk.load_library()
    ptr = ctypes.c_void_p(0x1000)
    E = (ctypes.c_float * 1)(0.05)
    big = sk.SkProblem(64, 2048, 2048, 32, 0, 0)  # about 390 MiB of workspace
    assert lib.sinkhorn_workspace_bytes(ctypes.byref(big)) > sk.SK_NOALLOC_MAX_BYTES
    assert lib.sinkhorn_solve_noalloc(ctypes.byref(big), ptr, ptr, ptr, ptr, E, 1, 5, ptr, ptr, None, None) == 6
    assert b"scratch" in lib.sinkhorn_last_error()
    small = sk.SkProblem(1, 100, 90, 3, 0, 0)
    assert lib.sinkhorn_solve_noalloc(ctypes.byref(small), None, ptr, ptr, ptr, E, 1, 5, ptr, ptr, None, None) == 1
    assert lib.sinkhorn_solve_noalloc(ctypes.byref(small), ptr, ptr, ptr, ptr, E, 1, -1, ptr, ptr, None, None) == 1
    assert lib.sinkhorn_solve_noalloc(ctypes.byref(sk.SkProblem(1, 0, 90, 3, 0, 0)), ptr, ptr, ptr, ptr, E, 1, 5,
                                      ptr, ptr, None, None) == 2


def _run_pair(p, eps):
    X, Y = torch.from_numpy(p.X).cuda(), torch.from_numpy(p.Y).cuda()
    a, b = torch.from_numpy(p.a).cuda(), torch.from_numpy(p.b).cuda()
    flags = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    f0, g0 = sk.solve_noalloc(X, Y, a, b, eps, p.iters, flags=flags)
    f1, g1 = sk.solve(X, Y, a, b, eps, p.iters)
    torch.cuda.synchronize()
    return f0, g0, f1, g1, int(flags.item())


@pytest.mark.gpu
def test_noalloc_matches_solve_twice_second_smaller():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sk.load_library()
    cases = [
        (make_case(1500, 1300, 16, seed=51, weights="softmax", scale=0.25, eps=0.05, iters=12), 0.05),
        (make_case(300, 200, 5, seed=52, weights="softmax", eps=0.1, iters=8), 0.1),
    ]
    for p, eps in cases:
        f0, g0, f1, g1, flags = _run_pair(p, eps)
        assert flags == 0, flags
        assert torch.equal(f0, f1) and torch.equal(g0, g1), "noalloc solve differs from sinkhorn_solve"
        rf, rg = oracle.solve(p.X[0], p.Y[0], p.a[0], p.b[0], eps, p.iters)
        ef = float(np.max(np.abs(f0[0].cpu().numpy() - rf)))
        eg = float(np.max(np.abs(g0[0].cpu().numpy() - rg)))
        assert ef <= _bound(eps, rf) and eg <= _bound(eps, rg), (ef, eg)
