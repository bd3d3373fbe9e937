"""Write full-trajectory oracle fixtures for the large workloads (CPU only).

For each workload this runs the fp64 oracle for the workload's full number of
iterations from f = g = 0 and stores the potentials at a seeded sample of
indices (plus the first and last index) as JSON under tests/golden/.  The GPU
parity tests compare the HIP path's potentials at those indices.

Only `oracle` and the seeded input generator are used: no value here comes from
the HIP path.  Runtime: workload 2 about three minutes, workload 3 about an hour
on 6 cores, workload 5 (all 64 problems) about a quarter of an hour.  For a
batched workload the indices run over the problem-major flattened potentials.

    python tests/golden/make_golden.py 2 3 [--threads N]
"""

from __future__ import annotations

import argparse
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
from log_domain_sinkhorn_half_amd.inputs import make_config  # noqa: E402

N_SAMPLE = 512


def digest(p) -> str:
    h = hashlib.sha256()
    for arr in (p.X, p.Y, p.a, p.b, p.eps):
        h.update(np.ascontiguousarray(arr).tobytes())
    return h.hexdigest()[:16]


def sample(n: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    idx = rng.choice(n, size=min(N_SAMPLE, n), replace=False)
    return np.unique(np.concatenate([idx, [0, n - 1]]))


def run(cfg: int, threads: int) -> str:
    p = make_config(cfg)
    eps = p.eps.astype(np.float64)
    t0 = time.time()
    if p.batch == 1:
        f, g = oracle.solve(p.X[0], p.Y[0], p.a[0], p.b[0], eps if eps.size > 1 else float(eps[0]),
                            p.iters, threads=threads)
        fi, gi = sample(p.n, 100 + cfg), sample(p.m, 200 + cfg)
    else:
        # batched workload: every problem, a few indices each (flattened problem-major)
        F, G = oracle.solve(p.X, p.Y, p.a, p.b, eps if eps.size > 1 else float(eps[0]), p.iters, threads=threads)
        f, g = F.reshape(-1), G.reshape(-1)
        fi, gi = sample(p.batch * p.n, 100 + cfg), sample(p.batch * p.m, 200 + cfg)
    dt = time.time() - t0
    out = {
        "workload": cfg,
        "name": p.name,
        "batch": p.batch,
        "iters": p.iters,
        "inputs_sha256_16": digest(p),
        "oracle_seconds": round(dt, 1),
        "oracle_threads": oracle.threads_used(threads),
        "f_index": fi.tolist(),
        "f": [float(v) for v in f[fi]],
        "g_index": gi.tolist(),
        "g": [float(v) for v in g[gi]],
        "f_absmax": float(np.max(np.abs(f))),
        "g_absmax": float(np.max(np.abs(g))),
    }
    path = os.path.join(HERE, f"trajectory_config{cfg}.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=0)
    return path


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("configs", type=int, nargs="+")
    ap.add_argument("--threads", type=int, default=0)
    a = ap.parse_args()
    for c in a.configs:
        print(run(c, a.threads), flush=True)


if __name__ == "__main__":
    main()
