"""Write the oracle fixture for Hessian-vector products whose conjugate-gradient
system spans several 2048-element blocks (CPU only).

Two seeded problems, eps = 0.2, d = 3, softmax weights:
  * "x": 48 moving points X against 4500 fixed points Y: the HVP in X solves a
    system in the 4500 potentials of Y (three blocks);
  * "y": 4500 points X against 48 moving points Y: the HVP in Y solves a system
    in the 4500 potentials of X (three blocks).
Potentials: 2000 oracle iterations from zero, rounded to fp32 (the GPU test
recomputes them the same way and checks their hash).  Direction V: seeded
normal draws.  The Hessian-vector products come from `oracle.hvp_x`, the dense
fp64 definition (the full (n+m) linear system solved by least squares), about a
minute each.  No value here comes from the HIP path.

    python tests/golden/make_hvp_golden.py
"""

from __future__ import annotations

import hashlib
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from log_domain_sinkhorn_half_amd.inputs import make_case  # noqa: E402

EPS = 0.2
ITERS = 2000
CASES = {"x": dict(n=48, m=4500, seed=301), "y": dict(n=4500, m=48, seed=302)}


def problem(side):
    c = CASES[side]
    return make_case(c["n"], c["m"], 3, seed=c["seed"], weights="softmax", eps=EPS)


def potentials(p):
    f, g = oracle.solve(p.X[0], p.Y[0], p.a[0], p.b[0], EPS, ITERS)
    return f.astype(np.float32), g.astype(np.float32)


def direction(side, p):
    rows = p.n if side == "x" else p.m
    return np.random.default_rng(CASES[side]["seed"] + 7).standard_normal((rows, 3)).astype(np.float32)


def pot_hash(f, g) -> str:
    return hashlib.sha256(f.tobytes() + g.tobytes()).hexdigest()[:16]


def main():
    out = {"eps": EPS, "iters": ITERS, "cases": {}}
    for side in ("x", "y"):
        t = time.time()
        p = problem(side)
        f, g = potentials(p)
        V = direction(side, p)
        X, Y, a, b = (np.asarray(v[0], np.float64) for v in (p.X, p.Y, p.a, p.b))
        if side == "x":
            hv = oracle.hvp_x(X, Y, a, b, f, g, EPS, V)
        else:
            hv = oracle.hvp_x(Y, X, b, a, g, f, EPS, V)
        out["cases"][side] = {**CASES[side], "potentials_sha256_16": pot_hash(f, g),
                              "hv": [[float(v) for v in row] for row in hv], "seconds": round(time.time() - t, 1)}
        print(side, "done", round(time.time() - t, 1), "s", flush=True)
    with open(os.path.join(HERE, "hvp_multiblock.json"), "w") as fh:
        json.dump(out, fh, indent=0)


if __name__ == "__main__":
    main()
