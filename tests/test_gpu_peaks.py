"""GPU: the peak rates the rooflines divide by, re-derived by microbenchmark.

The half-step's exp roofline uses 256 CUs x 4 SIMDs x 8 transcendental lanes x
2.4 GHz = 1.966e13 exp/s, and the MFMA rooflines AMD's dense 2516.6 (bf16) and
157.3 (fp32) TFLOP/s.  A measured rate well above one of these would mean the
roofline fraction is inflated; well below means the figure is not reachable
and the fractions understate the kernels.  Both are checked here, and the
measured rates are printed.
"""

import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["exp", "bf16", "fp32"])
def test_peak_rate_is_near_the_figure_the_roofline_uses(name):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from log_domain_sinkhorn_half_amd import peaks

    r = peaks.measure(name)
    print(f"{name}: measured {r['measured']:.4g}/s, roofline figure {r['spec']:.4g}/s, ratio {r['ratio']:.3f}")
    assert r["measured"] <= 1.05 * r["spec"], r
    assert r["measured"] >= 0.6 * r["spec"], r


def test_mixed_streams_are_slower_than_their_parts():
    """The exp rate with the half-steps' adds (and FMAs) in the same stream, and the
    d = 128 key-tile structure's MFMA rate: printed for the roofline discussion; each is
    bounded by the pure rate it shares a unit with."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from log_domain_sinkhorn_half_amd import peaks

    exp = peaks.measure("exp")["measured"]
    bf16 = peaks.measure("bf16")["measured"]
    for name, pure in (("exp+add", exp), ("fma+exp+add", exp), ("tile", bf16)):
        r = peaks.measure(name)
        print(f"{name}: {r['measured']:.4g}/s, {r['measured'] / pure:.3f} of the pure rate")
        assert 0.2 * pure <= r["measured"] <= 1.05 * pure, (name, r)
