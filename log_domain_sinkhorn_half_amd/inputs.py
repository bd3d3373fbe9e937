"""Seeded synthetic inputs for the log-domain Sinkhorn half-step path.

This module only draws random numbers and shapes them into problem instances;
it contains none of the Sinkhorn arithmetic.  The same arrays feed both the
fp64 CPU oracle and the HIP kernels, so parity tests compare like with like.

Every draw is made with numpy's PCG64 generator in float64 and then rounded to
float32 (round-to-nearest-even).  Half-precision inputs (``dtype="bf16"``) are
further rounded from float32 to bfloat16 with round-to-nearest-even; the
float32 array returned alongside holds exactly the bfloat16 values, so the
oracle sees the same numbers the kernels read.

The five named workloads (``make_config``) follow the benchmark settings of the
FlashSinkhorn summary (page "FlashSinkhorn: Trasporto Ottimo Entropico Consapevole delle I/O su GPU",
section "Risultati Sperimentali": synthetic point clouds, n up to ~70k), with
the shapes, distributions, epsilon and iteration counts fixed per workload.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = [
    "Problem",
    "CONFIG_NAMES",
    "make_config",
    "make_case",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "random_potential",
    "translate",
]


@dataclass
class Problem:
    """One (possibly batched) entropic OT instance.

    X: [B, n, d] float32 (for bf16 problems: the bf16 values, exactly, as float32)
    Y: [B, m, d] float32 (same convention)
    a: [B, n] float32 source weights; b: [B, m] float32 target weights
    eps: float32 array of length 1 (constant) or ``iters`` (a schedule)
    X_bits / Y_bits: uint16 bfloat16 bit patterns when dtype == "bf16", else None
    """

    name: str
    X: np.ndarray
    Y: np.ndarray
    a: np.ndarray
    b: np.ndarray
    eps: np.ndarray
    iters: int
    dtype: str = "fp32"
    X_bits: Optional[np.ndarray] = None
    Y_bits: Optional[np.ndarray] = None
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return self.X.shape[0]

    @property
    def n(self) -> int:
        return self.X.shape[1]

    @property
    def m(self) -> int:
        return self.Y.shape[1]

    @property
    def d(self) -> int:
        return self.X.shape[2]


# --------------------------------------------------------------------------
# bfloat16 rounding (round to nearest, ties to even), done on the bit pattern.
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (RNE); returns the uint16 bit patterns.

    NaN stays NaN (quiet); infinities stay infinite.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = ((u[nan] >> np.uint64(16)) | np.uint64(0x40)).astype(np.uint16)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to the float32 values they encode (exact)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# Building blocks
# --------------------------------------------------------------------------
def _softmax_weights(rng: np.random.Generator, shape) -> np.ndarray:
    z = rng.standard_normal(shape)
    z = z - z.max(axis=-1, keepdims=True)
    w = np.exp(z)
    w = w / w.sum(axis=-1, keepdims=True)
    return w.astype(np.float32)


def _uniform_weights(batch: int, n: int) -> np.ndarray:
    return np.full((batch, n), 1.0 / n, dtype=np.float32)


def _finish(name, X64, Y64, a, b, eps, iters, dtype, meta) -> Problem:
    X = np.ascontiguousarray(X64, dtype=np.float32)
    Y = np.ascontiguousarray(Y64, dtype=np.float32)
    X_bits = Y_bits = None
    if dtype == "bf16":
        X_bits = f32_to_bf16_bits(X)
        Y_bits = f32_to_bf16_bits(Y)
        X = bf16_bits_to_f32(X_bits).reshape(X.shape)
        Y = bf16_bits_to_f32(Y_bits).reshape(Y.shape)
        X_bits = X_bits.reshape(X.shape)
        Y_bits = Y_bits.reshape(Y.shape)
    elif dtype != "fp32":
        raise ValueError(f"unknown dtype {dtype!r}")
    eps = np.atleast_1d(np.asarray(eps, dtype=np.float64)).astype(np.float32)
    return Problem(name=name, X=X, Y=Y, a=np.ascontiguousarray(a, np.float32),
                   b=np.ascontiguousarray(b, np.float32), eps=eps, iters=int(iters),
                   dtype=dtype, X_bits=X_bits, Y_bits=Y_bits, meta=dict(meta))


def geometric_schedule(eps0: float, eps1: float, iters: int) -> np.ndarray:
    """eps_k = eps0 * (eps1/eps0)^(k/(iters-1)), k = 0..iters-1 (fp64)."""
    if iters == 1:
        return np.array([eps0], dtype=np.float64)
    k = np.arange(iters, dtype=np.float64)
    return eps0 * (eps1 / eps0) ** (k / (iters - 1))


# --------------------------------------------------------------------------
# The five named workloads
# --------------------------------------------------------------------------
CONFIG_NAMES = {
    1: "n=m=1024 d=3 fp32 eps=0.1 iters=20",
    2: "n=m=8192 d=64 fp32 eps=0.05 iters=100 softmax weights",
    3: "n=m=70000 d=3 fp32 eps=0.01 iters=200 cube vs 8-gaussian mixture",
    4: "n=65536 m=32768 d=128 bf16 eps=1.0->0.01 geometric iters=100",
    5: "batch=64 n=m=2048 d=32 fp32 eps=0.05 iters=50",
}


def make_config(k: int) -> Problem:
    """Build workload k (1..5) from seed k.  Draw order: X, Y, a, b."""
    rng = np.random.default_rng(k)
    if k == 1:
        n = m = 1024
        d = 3
        X = rng.standard_normal((1, n, d))
        Y = 0.5 + rng.standard_normal((1, m, d))
        a, b = _uniform_weights(1, n), _uniform_weights(1, m)
        return _finish("C1", X, Y, a, b, [0.1], 20, "fp32", {"config": 1})
    if k == 2:
        n = m = 8192
        d = 64
        X = rng.standard_normal((1, n, d)) / np.sqrt(d)
        Y = rng.standard_normal((1, m, d)) / np.sqrt(d)
        a = _softmax_weights(rng, (1, n))
        b = _softmax_weights(rng, (1, m))
        return _finish("C2", X, Y, a, b, [0.05], 100, "fp32", {"config": 2})
    if k == 3:
        n = m = 70000
        d = 3
        X = rng.random((1, n, d))
        means = rng.random((8, d))
        labels = rng.integers(0, 8, size=m)
        Y = (means[labels] + 0.05 * rng.standard_normal((m, d)))[None]
        a, b = _uniform_weights(1, n), _uniform_weights(1, m)
        return _finish("C3", X, Y, a, b, [0.01], 200, "fp32", {"config": 3})
    if k == 4:
        n, m, d = 65536, 32768, 128
        X = rng.standard_normal((1, n, d)) / np.sqrt(d)
        Y = rng.standard_normal((1, m, d)) / np.sqrt(d)
        a, b = _uniform_weights(1, n), _uniform_weights(1, m)
        eps = geometric_schedule(1.0, 0.01, 100)
        return _finish("C4", X, Y, a, b, eps, 100, "bf16", {"config": 4})
    if k == 5:
        B, n, m, d = 64, 2048, 2048, 32
        X = rng.standard_normal((B, n, d))
        mu = 0.5 * rng.standard_normal((B, 1, d))
        Y = mu + rng.standard_normal((B, m, d))
        a, b = _uniform_weights(B, n), _uniform_weights(B, m)
        return _finish("C5", X, Y, a, b, [0.05], 50, "fp32", {"config": 5})
    raise ValueError(f"no workload {k}; choose 1..5")


def make_case(n: int, m: int, d: int, *, batch: int = 1, eps=0.1, iters: int = 5,
              seed: int = 0, dtype: str = "fp32", weights: str = "uniform",
              dist: str = "gauss", shift: float = 0.5, scale: float = 1.0) -> Problem:
    """A small seeded instance for tests (same draw conventions as make_config).

    dist: "gauss"    X ~ N(0, s^2 I), Y ~ N(shift, s^2 I)
          "cube"     X, Y ~ U[0, s]^d
          "mixture"  X ~ U[0, s]^d, Y a mixture of 8 Gaussians of std 0.05 s with
                     means in U[0, s]^d (the shapes of the 70000-point workload)
    weights: "uniform" or "softmax" (softmax of i.i.d. N(0,1))
    """
    rng = np.random.default_rng(seed)
    if dist == "gauss":
        X = scale * rng.standard_normal((batch, n, d))
        Y = shift + scale * rng.standard_normal((batch, m, d))
    elif dist == "cube":
        X = scale * rng.random((batch, n, d))
        Y = scale * rng.random((batch, m, d))
    elif dist == "mixture":
        X = scale * rng.random((batch, n, d))
        means = scale * rng.random((batch, 8, d))
        labels = rng.integers(0, 8, size=(batch, m))
        Y = np.take_along_axis(means, labels[..., None], axis=1) + 0.05 * scale * rng.standard_normal((batch, m, d))
    else:
        raise ValueError(dist)
    if weights == "uniform":
        a, b = _uniform_weights(batch, n), _uniform_weights(batch, m)
    elif weights == "softmax":
        a, b = _softmax_weights(rng, (batch, n)), _softmax_weights(rng, (batch, m))
    else:
        raise ValueError(weights)
    return _finish(f"case{n}x{m}x{d}", X, Y, a, b, eps, iters, dtype,
                   {"seed": seed, "dist": dist})


def translate(p: Problem, t) -> Problem:
    """The same problem with both clouds moved by the vector t (a scalar moves every
    coordinate): x + t and y + t are formed in fp64 from the problem's values and
    rounded to its dtype again (round to nearest even), so the result is a new,
    exactly representable instance."""
    t = np.broadcast_to(np.asarray(t, dtype=np.float64), (p.d,))
    X = p.X.astype(np.float64) + t
    Y = p.Y.astype(np.float64) + t
    meta = dict(p.meta)
    meta["translate"] = t.tolist()
    return _finish(p.name + "+t", X, Y, p.a, p.b, p.eps.astype(np.float64), p.iters, p.dtype, meta)


def random_potential(shape, seed: int, scale: float = 1.0) -> np.ndarray:
    """A seeded float32 potential vector (used as a half-step input in tests)."""
    rng = np.random.default_rng(10_000 + seed)
    return (scale * rng.standard_normal(shape)).astype(np.float32)
