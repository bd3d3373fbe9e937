"""Benchmark: Sinkhorn iterations/s on one MI355X, with roofline and CPU-baseline legs.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3]

A step is one full Sinkhorn iteration (f half-step then g half-step) over the
workload, inputs resident in HBM.  The default workload is n = m = 70000,
d = 3, fp32, eps = 0.01 (X uniform in the unit cube, Y an 8-Gaussian
mixture), the scale the FlashSinkhorn summary calls the pain point (page
"FlashSinkhorn: Trasporto Ottimo Entropico Consapevole delle I/O su GPU", section "Enunciato del Problema").

Prints ONE JSON line.  The timed region is one sinkhorn_solve call of --steps
iterations (the product path: set-up, then fused half-steps that each write the
next one's key bias), continuing a trajectory after --warmup lead-in
iterations, after at least --min-warmup-s of untimed solves.  `roofline` covers
the dominant kernel (the streaming half-step kernel k_lse): its duration is the
timed solve's HIP-event time on the library's stream divided by its half-steps
(that window also holds the split merges and the amortised set-up; the
rocprofv3 summary under profiles/ separates them).  `cpu_baseline` times the
fp64 CPU oracle on a bounded row slice of the same workload on this host's cores.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Sinkhorn iters/sec & effective TFLOP/s at n=m=70000, fraction of roofline"

# MI355X peaks (AMD published figures; exp rate derived from unit counts and clock)
CLOCK_HZ = 2.4e9
N_CU = 256
PEAK_EXP_PER_S = N_CU * 4 * 8 * CLOCK_HZ       # 8 transcendental lanes/clk per SIMD, 4 SIMDs per CU
PEAK_MFMA = {"bf16": 2516.6e12, "fp32": 157.3e12}
PEAK_HBM = 8.0e12


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--min-warmup-s", type=float, default=1.5,
                    help="keep warming up (untimed iterations) until this much wall time has passed, "
                         "whatever --warmup says: a cold GPU reads slow for its first second or so")
    ap.add_argument("--config", type=int, default=3, help="workload 1..5 (default 3: n=m=70000, d=3)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-transport", action="store_true", help="skip the transport-application leg")
    ap.add_argument("--no-hvp", action="store_true", help="skip the Hessian-vector-product leg")
    ap.add_argument("--hvp-cg", type=int, default=50, help="CG iterations of the timed HVP")
    ap.add_argument("--cpu-seconds", type=float, default=6.0, help="target wall time of the CPU leg")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB mebibytes (scales rocprofv3 byte counters)")
    return ap.parse_args()


def kernel_source_hash() -> str:
    from log_domain_sinkhorn_half_amd.rocprof_harness import kernel_source_hash as code_hash
    return code_hash()


def read_traffic(kernel: str, workload: str):
    """Measured HBM bytes per launch from the committed rocprofv3 --pmc summary, or None
    if there is none or it was taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        line = line.strip().lstrip("-* ")
        if ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (got --gpus {args.gpus}); "
              "sharding across GPUs is not built", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n * 4, "launches": 3}), flush=True)
        return

    from log_domain_sinkhorn_half_amd import binding as sk
    from log_domain_sinkhorn_half_amd.inputs import make_config

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    sk.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    p = make_config(args.config)
    B, n, m, d = p.batch, p.n, p.m, p.d
    if p.dtype == "bf16":
        X = torch.from_numpy(p.X_bits.view(np.int16)).to(dev).view(torch.bfloat16)
        Y = torch.from_numpy(p.Y_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        X = torch.from_numpy(p.X).to(dev)
        Y = torch.from_numpy(p.Y).to(dev)
    a = torch.from_numpy(p.a).to(dev)
    b = torch.from_numpy(p.b).to(dev)
    ws = sk.alloc_workspace(X, Y)
    f = torch.zeros((B, n), dtype=torch.float32, device=dev)
    g = torch.zeros((B, m), dtype=torch.float32, device=dev)
    eps_sched = [float(e) for e in p.eps]

    def eps_at(k):
        return eps_sched[k % len(eps_sched)] if len(eps_sched) > 1 else eps_sched[0]

    K, W = args.steps, args.warmup

    def sched(k0, count):
        """eps of iterations k0 .. k0+count-1 (the schedule repeats past its end)."""
        if len(eps_sched) == 1:
            return eps_sched[0]
        return [eps_at(k) for k in range(k0, k0 + count)]

    # untimed warm-up: whole solves of max(W, 8) iterations until at least
    # --min-warmup-s of wall time has passed (each solve synchronises, so the
    # wall time is GPU time, not host run-ahead)
    t_warm = time.perf_counter()
    warm_iters = 0
    while warm_iters < W or time.perf_counter() - t_warm < args.min_warmup_s:
        it = max(W, 8)
        f.zero_()
        g.zero_()
        sk.solve(X, Y, a, b, sched(0, it), it, f=f, g=g, ws=ws)
        torch.cuda.synchronize()
        warm_iters += it
    warm_s = time.perf_counter() - t_warm
    # the timed steps continue a trajectory from f = g = 0 after W lead-in iterations
    f.zero_()
    g.zero_()
    if W > 0:
        sk.solve(X, Y, a, b, sched(0, W), W, f=f, g=g, ws=ws)
    torch.cuda.synchronize()

    # timed region: ONE sinkhorn_solve of K iterations (its set-up of norms,
    # centre and operands included), HIP events on the library's stream around it
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    sk.solve(X, Y, a, b, sched(W, K), K, f=f, g=g, ws=ws)
    ev1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    solve_ms = ev0.elapsed_time(ev1)
    assert torch.isfinite(f).all() and torch.isfinite(g).all(), "non-finite potentials"
    flags = sk.range_flags(X, Y, ws)

    # side measurement (not the headline): the same iterations as standalone
    # half-step calls, each preparing its key operand, with events per half-step
    M = min(K, 10)
    f2, g2 = f.clone(), g.clone()
    evh = [torch.cuda.Event(enable_timing=True) for _ in range(2 * M + 1)]
    torch.cuda.synchronize()
    evh[0].record(stream)
    for k in range(M):
        e = eps_at(W + k)
        sk.half_step_f(X, Y, ws, g2, e, f=f2)
        evh[2 * k + 1].record(stream)
        sk.half_step_g(X, Y, ws, f2, e, g=g2)
        evh[2 * k + 2].record(stream)
    torch.cuda.synchronize()
    half_ms = np.array([evh[i].elapsed_time(evh[i + 1]) for i in range(2 * M)])
    f_ms, g_ms = half_ms[0::2], half_ms[1::2]

    iters_per_s = K / elapsed
    ms_per_step = 1e3 * elapsed / K
    elems_iter = 2.0 * B * n * m                      # score elements (= exps) per iteration
    eff_ops_iter = 4.0 * B * n * m * d + 2.0 * B * n * m
    eff_tflops = eff_ops_iter * iters_per_s / 1e12
    contraction = "bf16" if p.dtype == "bf16" else "fp32"
    t_exp = elems_iter / PEAK_EXP_PER_S
    t_mfma = 4.0 * B * n * m * d / PEAK_MFMA[contraction]
    bound = "alu" if t_exp >= t_mfma else "mfma"
    t_roof = max(t_exp, t_mfma)
    frac_iter = t_roof / (elapsed / K)

    # dominant kernel: one half-step launch processes B*n*m (f) or B*m*n (g) score
    # elements; its duration is taken as the timed solve's event time over its 2K
    # half-steps (which also holds the split merges and the amortised set-up, so
    # the fraction errs low; the rocprofv3 summary gives the kernel alone)
    launch_s = solve_ms / (2 * K) / 1e3
    elems_launch = B * n * m
    workload = f"C{args.config}"
    traffic = read_traffic("k_lse", workload)
    if bound == "alu":
        achieved = elems_launch / launch_s / 1e9
        roof = {"bound": "alu", "achieved": round(achieved, 1), "peak": round(PEAK_EXP_PER_S / 1e9, 1),
                "unit": "Gexp/s", "frac": round(achieved * 1e9 / PEAK_EXP_PER_S, 4)}
    else:
        achieved = 2.0 * d * elems_launch / launch_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_MFMA[contraction] / 1e12,
                "unit": "TFLOP/s", "frac": round(achieved * 1e12 / PEAK_MFMA[contraction], 4)}
    if bound == "mfma" and contraction == "fp32":
        # fp32 scores come from exact bf16 splits on the bf16 matrix cores; the same
        # algorithmic flops priced at a third of the bf16 peak (a 3-product split)
        roof["vs_bf16_3pass"] = {"path": "fp32 scores from exact bf16 operand splits on bf16 MFMA",
                                 "peak": round(PEAK_MFMA["bf16"] / 3 / 1e12, 1),
                                 "frac": round(achieved * 1e12 / (PEAK_MFMA["bf16"] / 3), 4)}
    roof["traffic"] = traffic
    roof["launch_ms"] = round(launch_s * 1e3, 4)
    roof["window"] = f"one sinkhorn_solve of {K} iterations, HIP events on its stream, per half-step"

    out = {
        "metric": METRIC,
        "value": round(iters_per_s, 2),
        "unit": "iters/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if p.dtype == "fp32" else "bf16",
        "data": "synthetic (seeded generator log_domain_sinkhorn_half_amd/inputs.py)",
        "config": {"workload": f"C{args.config}: {p.name} batch={B} n={n} m={m} d={d} {p.dtype} "
                               f"eps={eps_sched[0] if len(eps_sched) == 1 else 'schedule'}",
                   "batch": B, "n": n, "m": m, "d": d, "parallelism": "single GPU"},
        "effective_tflops": round(eff_tflops, 3),
        "roofline_frac_per_iteration": round(frac_iter, 4),
        "solve_event_ms": round(solve_ms, 4),
        "range_flags": flags,
        "standalone_half_steps": {
            "what": f"{M} iterations as half_step_f / half_step_g calls, each preparing its key operand",
            "half_step_ms": {"f": round(float(np.mean(f_ms)), 4), "g": round(float(np.mean(g_ms)), 4)},
            "iters_per_s": round(1e3 / float(np.sum(half_ms) / M), 2)},
        "roofline": roof,
        "warmup_done": {"iterations": warm_iters, "seconds": round(warm_s, 3),
                        "rule": f"max(--warmup, {args.min_warmup_s} s of iterations), then the trajectory restarts "
                                f"and --warmup iterations lead into the timed steps"},
        "gpu_clock_mhz": gpu_clock_mhz(),
    }

    if not args.no_transport:
        out["transport"] = transport_leg(sk, X, Y, a, b, f, g, eps_sched[-1], p, contraction)
    if not args.no_hvp:
        out["hvp"] = hvp_leg(sk, X, Y, a, b, f, g, eps_sched[-1], p, args.hvp_cg, contraction)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(p, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def gpu_clock_mhz():
    """Current and highest graphics clock of GPU 0 in MHz from amd-smi's Python
    module, read right after the timed steps (None where it cannot be read)."""
    try:
        import amdsmi

        amdsmi.amdsmi_init()
        try:
            h = amdsmi.amdsmi_get_processor_handles()[0]
            info = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX)
            keep = ("clk", "cur_clk", "max_clk", "min_clk", "clk_locked", "clk_deep_sleep")
            return {k: v for k, v in info.items() if k in keep}
        finally:
            amdsmi.amdsmi_shut_down()
    except Exception as e:  # noqa: BLE001 - the clock is a report, never a failure
        return {"unavailable": type(e).__name__}


def warm_for(call, seconds):
    """Repeat `call` (GPU work) until `seconds` of wall time have passed."""
    import time

    import torch

    t0 = time.perf_counter()
    while True:
        call()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return


def transport_leg(sk, X, Y, a, b, f, g, eps, p, contraction, reps=10):
    """Time the transport application (barycentric projection + gradient) of each
    side at the final potentials.  One call = key preparation plus one streaming
    P.V pass with lazy row offsets: 1 exp and 4d algorithmic flops (the score
    contraction and P.V) per score element."""
    import numpy as np
    import torch

    ws = sk.alloc_workspace(X, Y, transport=True)
    sk.init_norms(X, Y, a, b, ws)
    bx, gx = sk.barycentric_x(X, Y, ws, f, g, eps)
    by, gy = sk.barycentric_y(X, Y, ws, f, g, eps)
    torch.cuda.synchronize()
    # the GPU idles while the CPU leg runs: bring it back to its clock first
    warm_for(lambda: (sk.barycentric_x(X, Y, ws, f, g, eps, bary=bx, grad=gx),
                      sk.barycentric_y(X, Y, ws, f, g, eps, bary=by, grad=gy)), 0.3)
    stream = torch.cuda.current_stream()
    ms = {}
    for side, call, outs in (("x", sk.barycentric_x, (bx, gx)), ("y", sk.barycentric_y, (by, gy))):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record(stream)
        for r in range(reps):
            call(X, Y, ws, f, g, eps, bary=outs[0], grad=outs[1])
            ev[r + 1].record(stream)
        torch.cuda.synchronize()
        ms[side] = float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]))
    assert all(torch.isfinite(t).all() for t in (bx, gx, by, gy)), "non-finite transport outputs"
    elems = p.batch * p.n * p.m
    t_call = 0.5 * (ms["x"] + ms["y"]) / 1e3
    t_exp = 1.0 * elems / PEAK_EXP_PER_S
    t_mfma = 4.0 * elems * p.d / PEAK_MFMA[contraction]
    if t_exp >= t_mfma:
        roof = {"bound": "alu", "achieved": round(1.0 * elems / t_call / 1e9, 1),
                "peak": round(PEAK_EXP_PER_S / 1e9, 1), "unit": "Gexp/s", "frac": round(t_exp / t_call, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(4.0 * elems * p.d / t_call / 1e12, 2),
                "peak": PEAK_MFMA[contraction] / 1e12, "unit": "TFLOP/s", "frac": round(t_mfma / t_call, 4)}
    return {"what": "barycentric projection + gradient of every point (one call per side)",
            "ms_per_call": {"x": round(ms["x"], 4), "y": round(ms["y"], 4)}, "reps": reps, "roofline": roof}


def hvp_leg(sk, X, Y, a, b, f, g, eps, p, cg_iters, contraction, reps=3):
    """Time one Hessian-vector product in X (fixed CG iteration count, no early stop).
    Every plan pass evaluates each of the B*n*m scores once: 2 half-steps, the plan
    applied to Y, P^T [z, v, cr/r], 2 passes per CG iteration, P [dg, dg y] (each
    plan product takes ceil(columns / 64) passes) and one row-weighted pass for the
    quadratic term sum_j P_ij (y_j . v_i) y_j."""
    import math

    import numpy as np
    import torch

    ws = sk.alloc_workspace(X, Y, hvp=True)
    sk.init_norms(X, Y, a, b, ws)
    gen = torch.Generator(device="cuda").manual_seed(0)
    V = torch.randn((p.batch, p.n, p.d), device="cuda", generator=gen)
    out = sk.hvp_x(X, Y, ws, f, g, eps, V, cg_iters=cg_iters, cg_tol=0.0)
    torch.cuda.synchronize()
    warm_for(lambda: sk.hvp_x(X, Y, ws, f, g, eps, V, cg_iters=cg_iters, cg_tol=0.0, out=out), 0.3)
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(stream)
    for r in range(reps):
        sk.hvp_x(X, Y, ws, f, g, eps, V, cg_iters=cg_iters, cg_tol=0.0, out=out)
        ev[r + 1].record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]))
    assert torch.isfinite(out).all(), "non-finite HVP"
    d = p.d
    passes = 2 + math.ceil(d / 64) + math.ceil((d + 2) / 64) + 2 * cg_iters + math.ceil((d + 1) / 64) + 1
    nm = p.batch * p.n * p.m
    exps = passes * nm
    # algorithmic flops per score of each pass: the score contraction (2d) plus the
    # plan product over its columns (2c), and for the quadratic term the direction's
    # contraction too (2d + 2d + 2d)
    def plan(c):  # ceil(c / 64) passes, each scoring every pair, and 2c flops of plan product
        return math.ceil(c / 64) * 2 * d + 2 * c
    flops = nm * (2 * 2 * d + plan(d) + plan(d + 2) + 2 * cg_iters * plan(1) + plan(d + 1) + 6 * d)
    t_call = ms / 1e3
    t_exp = exps / PEAK_EXP_PER_S
    t_mfma = flops / PEAK_MFMA[contraction]
    if t_exp >= t_mfma:
        roof = {"bound": "alu", "achieved": round(exps / t_call / 1e9, 1), "peak": round(PEAK_EXP_PER_S / 1e9, 1),
                "unit": "Gexp/s", "frac": round(t_exp / t_call, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(flops / t_call / 1e12, 2), "peak": PEAK_MFMA[contraction] / 1e12,
                "unit": "TFLOP/s", "frac": round(t_mfma / t_call, 4)}
    return {"what": f"one Hessian-vector product in X, {cg_iters} CG iterations ({passes} plan passes)",
            "ms_per_call": round(ms, 3), "reps": reps, "roofline": roof}


def cpu_baseline(p, target_s: float):
    """fp64 oracle (as it stands) on a row slice: f half-step for r rows of X against all
    of Y, then g half-step for r rows of Y against all of X (problem 0), extrapolated to a
    full iteration of the whole workload."""
    import numpy as np

    import oracle
    from log_domain_sinkhorn_half_amd.inputs import random_potential

    threads = len(os.sched_getaffinity(0))
    used = oracle.threads_used(threads)
    X, Y, a, b = (np.asarray(v[0], np.float64) for v in (p.X, p.Y, p.a, p.b))
    g = random_potential(p.m, 99, 0.1).astype(np.float64)
    f = random_potential(p.n, 98, 0.1).astype(np.float64)
    eps = float(p.eps[-1])

    def run(r):
        rows_x = np.arange(min(r, p.n))
        rows_y = np.arange(min(r, p.m))
        t = time.perf_counter()
        oracle.half_step_f(X, Y, b, g, eps, rows=rows_x, threads=used)
        oracle.half_step_g(X, Y, a, f, eps, rows=rows_y, threads=used)
        return time.perf_counter() - t, rows_x.size, rows_y.size

    r = 256
    dt, rx, ry = run(r)
    while dt < 0.25 * target_s and (rx < p.n or ry < p.m):
        r = int(min(max(p.n, p.m), r * max(2.0, 0.5 * target_s / max(dt, 1e-3))))
        dt, rx, ry = run(r)
    # work-proportional: the slice evaluated rx*m + ry*n cost terms, a full
    # iteration of every problem evaluates 2*n*m per problem
    t_iter = p.batch * dt * (2.0 * p.n * p.m) / (rx * p.m + ry * p.n)
    return {"value": round(1.0 / t_iter, 6), "unit": "iters/s", "cores": used, "kind": "oracle",
            "sample": f"one f half-step over {rx} rows of X and one g half-step over {ry} rows of Y "
                      f"(problem 0, all {p.m}/{p.n} points on the other side), {dt:.2f} s wall, "
                      f"extrapolated linearly to {p.batch} x ({p.n}+{p.m}) rows"}


if __name__ == "__main__":
    main()
