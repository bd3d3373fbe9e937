"""Write full-trajectory oracle fixtures for the large workloads (CPU only).

For each workload this runs the fp64 oracle for the workload's full number of
iterations from f = g = 0 and stores the potentials at a seeded sample of
indices (plus the first and last index) as JSON under tests/golden/.  The GPU
parity tests compare the HIP path's potentials at those indices.

With ``--per-iter K`` (single problems only) the fixture also holds, for every
iteration k, the potentials f_k and g_k at K seeded indices per side, so that a
test can check each of the trajectory's half-steps, not only the last.  The
oracle then runs one iteration per call, carrying g between calls, which is the
same loop as a single call (the f half-step reads only the incoming g).

Only `oracle` and the seeded input generator are used: no value here comes from
the HIP path.  Runtime: workload 2 (8192^2, d = 64) about three minutes,
workload 3 (70000^2, d = 3) about an hour on 6 cores, workload 4 (65536 x 32768,
d = 128, bf16) about three hours on 8 cores, workload 5 (64 problems of 2048^2,
d = 32) about a quarter of an hour.  For a batched workload the indices run
over the problem-major flattened potentials.

    python tests/golden/make_golden.py 2 3 [--threads N]
    python tests/golden/make_golden.py 4 --per-iter 64 [--checkpoint PATH.npz]
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


def sample(n: int, seed: int, k: int = N_SAMPLE) -> np.ndarray:
    rng = np.random.default_rng(seed)
    idx = rng.choice(n, size=min(k, n), replace=False)
    return np.unique(np.concatenate([idx, [0, n - 1]]))


def _per_iter_solve(p, eps, threads, fi_k, gi_k, checkpoint):
    """One oracle iteration per call; returns final (f, g) and the sampled history."""
    X, Y, a, b = p.X[0], p.Y[0], p.a[0], p.b[0]
    g = np.zeros(p.m, dtype=np.float64)
    f = np.zeros(p.n, dtype=np.float64)
    hist_f, hist_g, k0 = [], [], 0
    if checkpoint and os.path.exists(checkpoint):
        ck = np.load(checkpoint)
        if ck["digest"].item() == digest(p):
            f, g = ck["f"], ck["g"]
            hist_f, hist_g = list(ck["hist_f"]), list(ck["hist_g"])
            k0 = len(hist_f)
            print(f"resuming at iteration {k0}", flush=True)
    for k in range(k0, p.iters):
        e = float(eps[k] if eps.size > 1 else eps[0])
        t0 = time.time()
        f, g = oracle.solve(X, Y, a, b, e, 1, g0=g, threads=threads)
        hist_f.append(f[fi_k].copy())
        hist_g.append(g[gi_k].copy())
        if checkpoint:
            tmp = checkpoint + ".tmp.npz"
            np.savez(tmp, digest=np.array(digest(p)), f=f, g=g, hist_f=np.array(hist_f), hist_g=np.array(hist_g))
            os.replace(tmp, checkpoint)
        print(f"iteration {k} eps {e:.6g} {time.time() - t0:.1f} s", flush=True)
    return f, g, np.array(hist_f), np.array(hist_g)


def run(cfg: int, threads: int, per_iter: int = 0, checkpoint: str = "") -> str:
    p = make_config(cfg)
    eps = p.eps.astype(np.float64)
    t0 = time.time()
    extra = {}
    if p.batch == 1 and per_iter > 0:
        fi_k, gi_k = sample(p.n, 300 + cfg, per_iter), sample(p.m, 400 + cfg, per_iter)
        f, g, hf, hg = _per_iter_solve(p, eps, threads, fi_k, gi_k, checkpoint)
        fi, gi = sample(p.n, 100 + cfg), sample(p.m, 200 + cfg)
        extra = {
            "per_iter_f_index": fi_k.tolist(),
            "per_iter_g_index": gi_k.tolist(),
            "per_iter_f": [[float(v) for v in row] for row in hf],
            "per_iter_g": [[float(v) for v in row] for row in hg],
            "per_iter_f_absmax": [float(np.max(np.abs(r))) for r in hf],
        }
    elif p.batch == 1:
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
    out.update(extra)
    path = os.path.join(HERE, f"trajectory_config{cfg}.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=0)
    return path


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("configs", type=int, nargs="+")
    ap.add_argument("--threads", type=int, default=0)
    ap.add_argument("--per-iter", type=int, default=0,
                    help="also store f_k, g_k at this many indices per side for every iteration")
    ap.add_argument("--checkpoint", default="", help="npz file to resume a per-iteration run from")
    a = ap.parse_args()
    for c in a.configs:
        print(run(c, a.threads, a.per_iter, a.checkpoint), flush=True)


if __name__ == "__main__":
    main()
