"""The Python binding rejects wrongly shaped or placed tensors before any launch.

The C ABI receives raw pointers and sizes taken from X and Y only, so the
binding is the one place that can tell that f, g, a weight vector, a value
matrix or an output does not match the problem.  These checks run before the
library is loaded or any device is touched, so they are tested on the CPU.
"""

import pytest
import torch

from log_domain_sinkhorn_half_amd import binding as sk

B, N, M, D = 2, 5, 7, 3


def clouds():
    return torch.zeros(B, N, D), torch.zeros(B, M, D)


def vec(*shape):
    return torch.zeros(*shape)


WS = torch.zeros(16, dtype=torch.uint8)


@pytest.mark.parametrize("call", [
    lambda X, Y: sk.init_norms(X, Y, vec(B, N + 1), vec(B, M), WS),
    lambda X, Y: sk.init_norms(X, Y, vec(B, N), vec(M), WS),
    lambda X, Y: sk.half_step_f(X, Y, WS, vec(B, N), 0.1),
    lambda X, Y: sk.half_step_f(X, Y, WS, vec(B, M), 0.1, f=vec(B, M)),
    lambda X, Y: sk.half_step_g(X, Y, WS, vec(B, M), 0.1),
    lambda X, Y: sk.solve(X, Y, vec(B, N), vec(B, M), 0.1, 3, g=vec(1, M)),
    lambda X, Y: sk.solve(X, Y, vec(B, M), vec(B, M), 0.1, 3),
    lambda X, Y: sk.marginal_error(X, Y, WS, vec(B, N), vec(B, M), 0.1, err=vec(B, 3)),
    lambda X, Y: sk.barycentric_x(X, Y, WS, vec(B, N), vec(B, M), 0.1, bary=vec(B, M, D)),
    lambda X, Y: sk.barycentric_y(X, Y, WS, vec(B, N), vec(B, M), 0.1, grad=vec(B, M, D + 1)),
    lambda X, Y: sk.apply_plan_x(X, Y, WS, vec(B, N), vec(B, M), 0.1, vec(B, N, 4)),
    lambda X, Y: sk.apply_plan_x(X, Y, WS, vec(B, N), vec(B, M), 0.1, vec(B, M, 4), out=vec(B, M, 4)),
    lambda X, Y: sk.apply_plan_y(X, Y, WS, vec(B, N), vec(B, M), 0.1, vec(B, M)),
    lambda X, Y: sk.hvp_x(X, Y, WS, vec(B, N), vec(B, M), 0.1, vec(B, M, D)),
    lambda X, Y: sk.hvp_y(X, Y, WS, vec(B, N), vec(B, M), 0.1, vec(B, M, D), out=vec(B, N, D)),
])
def test_wrong_shape_raises_before_launch(call):
    X, Y = clouds()
    with pytest.raises(ValueError, match="shape"):
        call(X, Y)


def test_single_problem_may_drop_the_batch_axis():
    X, Y = torch.zeros(N, D), torch.zeros(M, D)
    # shapes are right ([n] for a [1, n] weight vector), so the first complaint is the device
    with pytest.raises(ValueError, match="device tensor"):
        sk.init_norms(X, Y, vec(N), vec(M), WS)


def test_mismatched_clouds_raise():
    with pytest.raises(ValueError):
        sk.problem_of(torch.zeros(B, N, D), torch.zeros(B, M, D + 1))
    with pytest.raises(ValueError):
        sk.problem_of(torch.zeros(B, N, D), torch.zeros(B + 1, M, D))
