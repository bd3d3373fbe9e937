"""GPU: the solve under HIP graph capture.

Every call of the library only enqueues kernels on the caller's stream (no
allocation, copy, memset or synchronisation), so a caller may capture a whole
`sinkhorn_solve` (or the allocation-free `sinkhorn_solve_noalloc`) in a graph
and replay it.  Each replay here runs after eager work on the same buffers and
must reproduce the eager solve bit for bit (replays of graphs holding memset
nodes have been seen to go wrong after the first, so several are checked).
"""

import numpy as np
import pytest
import torch

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


@pytest.mark.parametrize("noalloc", [False, True])
@pytest.mark.parametrize("n,m,d,dtype,batch,annealed", [(700, 500, 3, "fp32", 1, False), (300, 520, 64, "bf16", 1, True),
                                                        (257, 300, 32, "fp32", 3, False), (150, 200, 130, "fp32", 1, True)])
def test_captured_solve_replays_match_eager(n, m, d, dtype, batch, annealed, noalloc):
    p = make_case(n, m, d, batch=batch, seed=n + d, weights="softmax", dtype=dtype, scale=1.0 / np.sqrt(d))
    X, Y, a, b = dev(p)
    iters = 6
    eps = (0.5 * 0.2 ** (np.arange(iters) / (iters - 1))).astype(np.float32).tolist() if annealed else 0.1
    ws = None if noalloc else sk.alloc_workspace(X, Y)
    f = torch.zeros((batch, n), device="cuda")
    g = torch.zeros((batch, m), device="cuda")

    def solve():
        if noalloc:
            sk.solve_noalloc(X, Y, a, b, eps, iters, f=f, g=g)
        else:
            sk.solve(X, Y, a, b, eps, iters, f=f, g=g, ws=ws)

    # eager reference (twice: the second run sees every cache the first one filled)
    for _ in range(2):
        f.zero_()
        g.zero_()
        solve()
    torch.cuda.synchronize()
    ref_f, ref_g = f.clone(), g.clone()

    graph = torch.cuda.CUDAGraph()
    f.zero_()
    g.zero_()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        solve()
    for r in range(3):
        f.zero_()
        g.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(f, ref_f) and torch.equal(g, ref_g), f"replay {r} differs from the eager solve"
        # eager work on the same buffers between replays
        f.zero_()
        g.zero_()
        solve()
        torch.cuda.synchronize()
        assert torch.equal(f, ref_f) and torch.equal(g, ref_g), f"eager solve after replay {r} differs"
    del graph
