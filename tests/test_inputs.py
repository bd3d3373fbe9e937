"""The seeded input generator: determinism, shapes, and bf16 rounding."""

import numpy as np
import pytest
import torch

from log_domain_sinkhorn_half_amd.inputs import (bf16_bits_to_f32, f32_to_bf16_bits, make_case,
                                                 make_config)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 65504.0, 1e-40, -3.4e38, np.inf, -np.inf],
                                 np.float32)])
    # ties: values exactly half-way between two bf16 numbers
    ties = (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties])
    bits = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)
    back = bf16_bits_to_f32(bits)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_small_case_is_deterministic():
    p1 = make_case(33, 17, 5, seed=4, weights="softmax")
    p2 = make_case(33, 17, 5, seed=4, weights="softmax")
    for k in ("X", "Y", "a", "b", "eps"):
        np.testing.assert_array_equal(getattr(p1, k), getattr(p2, k))
    assert p1.X.dtype == np.float32 and p1.X.shape == (1, 33, 5)
    assert abs(p1.a.sum() - 1) < 1e-5 and abs(p1.b.sum() - 1) < 1e-5


@pytest.mark.parametrize("k,shape", [(1, (1, 1024, 1024, 3)), (5, (64, 2048, 2048, 32))])
def test_config_shapes(k, shape):
    p = make_config(k)
    assert (p.batch, p.n, p.m, p.d) == shape
    assert p.X.flags.c_contiguous and p.Y.flags.c_contiguous


def test_config4_is_bf16_with_geometric_schedule():
    p = make_config(4)
    assert p.dtype == "bf16" and p.X_bits.dtype == np.uint16
    np.testing.assert_array_equal(bf16_bits_to_f32(p.X_bits).reshape(p.X.shape), p.X)
    assert p.eps.shape == (100,)
    assert p.eps[0] == np.float32(1.0) and p.eps[-1] == np.float32(0.01)
    r = p.eps[1:].astype(np.float64) / p.eps[:-1]
    np.testing.assert_allclose(r, (0.01) ** (1 / 99), rtol=1e-6)


def test_config3_mixture_structure():
    p = make_config(3)
    assert p.X.min() >= 0 and p.X.max() <= 1
    # 8 tight clusters: every target point is within 6 std of one of 8 centres
    assert p.Y.shape == (1, 70000, 3)
    assert p.eps[0] == np.float32(0.01) and p.iters == 200
