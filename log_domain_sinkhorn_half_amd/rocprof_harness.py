"""rocprofv3 harness for the streaming half-step kernel (k_lse) on one workload.

    python -m log_domain_sinkhorn_half_amd.rocprof_harness --config 3 --out rocprof_out/rp [--write-profiles]
        [--kernel k_bary]

Runs `bench.py` under rocprofv3 in separate passes and summarises, per launch of
k_lse (or of the kernel named by --kernel, e.g. the transport pass k_bary, whose
counter passes then keep the benchmark's transport leg):
  * duration (kernel trace, the default benchmark command without its CPU leg);
  * MFMA utilisation (busy cycles of the matrix cores over all SIMDs) and the
    executed bf16 MFMA rate against the 2516.6 TFLOP/s dense peak;
  * transcendental (v_exp_f32) rate against the exp peak of 256 CUs x 4 SIMDs x
    8 lanes x 2.4 GHz, and VALU instructions per SIMD cycle;
  * LDS use: busy fraction, bank-conflict cycles, and the share of wave time
    spent waiting on LDS or on any counter;
  * HBM traffic (FETCH_SIZE and WRITE_SIZE, each in a pass of its own, scaled by
    what the same counter reads for a plain 256 MiB device copy) and GB/s.

Counter passes respect the per-block limits of one rocprofv3 run (at most 8 SQ
and 2 GRBM counters; FETCH_SIZE and WRITE_SIZE alone) and run under
`timeout -s KILL`.  This process never touches the GPU: every GPU step is a
child process.  With --write-profiles the summaries replace
profiles/k_lse_C<k>_{kernel_trace,traffic,counters}.md; the traffic file carries
the kernel source hash that bench.py checks before reporting `traffic`.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# MI355X (gfx950) figures used to normalise counters
N_XCC = 8
N_CU = 256
N_SIMD = 4 * N_CU
CLOCK_HZ = 2.4e9
PEAK_BF16 = 2516.6e12
PEAK_EXP = N_SIMD * 8 * CLOCK_HZ
PEAK_HBM = 8.0e12

SQ_PASS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_VALU",
           "SQ_INSTS_MFMA", "SQ_ACTIVE_INST_VALU", "SQ_BUSY_CU_CYCLES", "SQ_WAVES", "GRBM_GUI_ACTIVE"]
LDS_PASS = ["SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS", "SQ_WAIT_INST_LDS", "SQ_WAIT_ANY",
            "SQ_WAVE_CYCLES", "SQ_INSTS_SALU", "SQ_ACTIVE_INST_LDS", "GRBM_GUI_ACTIVE"]

DESC = {1: "n=m=1024, d=3, fp32, eps=0.1", 2: "n=m=8192, d=64, fp32, eps=0.05", 3: "n=m=70000, d=3, fp32, eps=0.01",
        4: "n=65536, m=32768, d=128, bf16, eps 1.0 -> 0.01", 5: "batch 64, n=m=2048, d=32, fp32, eps=0.05"}
# (batch, n, m, d, bf16 inputs) of the workloads
SHAPE = {1: (1, 1024, 1024, 3, False), 2: (1, 8192, 8192, 64, False), 3: (1, 70000, 70000, 3, False),
         4: (1, 65536, 32768, 128, True), 5: (64, 2048, 2048, 32, False)}


def operand_slots(d: int, bf16: bool) -> int:
    """K slots per point of the half-step operands: d rounded up to 32 for bf16
    inputs; for fp32 inputs the grid section (d + 5 slots) and 7d + 2 correction
    slots, each section on a 32-slot boundary unless both fit one (d <= 3)."""
    if bf16:
        return (d + 31) // 32 * 32
    grid, corr = d + 5, 7 * d + 2
    if grid <= 8 and corr <= 24:
        return 32
    cb = (grid + 31) // 32 * 32
    return (cb + corr + 31) // 32 * 32


def algorithmic_bytes(C: int) -> float:
    """Algorithmic HBM bytes of one half-step launch, averaged over the f and g
    launches: half of an iteration's 2 (n+m) d s + 20 (n+m) bytes per problem
    (both clouds read once at s bytes per coordinate; potentials, weights and
    norms: 20 bytes per point), the figure the roofline tables use."""
    B, n, m, d, bf16 = SHAPE[C]
    s = 2 if bf16 else 4
    return B * ((n + m) * d * s + 10 * (n + m))


def operand_bytes(C: int) -> float:
    """Bytes of the kernel's own operand rows read once per half-step launch (K
    slots of 2 bytes per point of both sides, averaged), plus the potential."""
    B, n, m, d, bf16 = SHAPE[C]
    kp = operand_slots(d, bf16)
    return B * (n + m) * kp * 2 + B * (n + m) / 2 * 4


def code_hash(src: str) -> str:
    """Hash of C/C++ source with comments and whitespace left out."""
    code = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    code = re.sub(r"//[^\n]*", " ", code)
    return hashlib.sha256(" ".join(code.split()).encode()).hexdigest()[:16]


def kernel_source_hash() -> str:
    """Hash of the kernel source's code, so a summary stays tied to the code it
    measured and survives comment edits."""
    return code_hash(open(os.path.join(ROOT, "log_domain_sinkhorn_half_amd", "csrc", "sinkhorn.hip")).read())


def short(name: str) -> str:
    return name.replace("void ", "").replace("(anonymous namespace)::", "").split("(")[0]


def run(cmd: list, log: str, what: str) -> None:
    print(f"[harness] {what}: {' '.join(cmd)}", flush=True)
    with open(log, "w") as fh:
        rc = subprocess.run(cmd, cwd=ROOT, stdout=fh, stderr=subprocess.STDOUT).returncode
    if rc != 0:
        tail = open(log).read()[-2000:]
        raise SystemExit(f"[harness] {what} failed with status {rc}; log {log}:\n{tail}")
    print(f"[harness] {what}: done", flush=True)


def counters(path_glob: str, kernel: str) -> dict:
    """Mean per dispatch of every counter over the dispatches whose name contains `kernel`."""
    files = glob.glob(path_glob, recursive=True)
    if not files:
        raise SystemExit(f"[harness] no counter file matches {path_glob}")
    acc: dict = {}
    for r in csv.DictReader(open(files[0])):
        if kernel in r["Kernel_Name"]:
            acc.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--out", default="rocprof_out")
    ap.add_argument("--steps", type=int, default=5, help="timed steps of the counter passes")
    ap.add_argument("--write-profiles", action="store_true")
    ap.add_argument("--summarize-only", action="store_true", help="reuse the outputs already under --out")
    ap.add_argument("--kernel", default="k_lse", help="kernel name (prefix) to summarise")
    args = ap.parse_args()
    C = args.config
    out = os.path.abspath(args.out)
    os.makedirs(out, exist_ok=True)
    os.environ.setdefault("TMPDIR", "/tmp")
    py = sys.executable
    bench = [py, "bench.py", "--config", str(C)]
    kname = args.kernel
    short_bench = bench + ["--steps", str(args.steps), "--warmup", "2", "--no-cpu-baseline", "--no-hvp"]
    if kname == "k_lse":
        short_bench.append("--no-transport")
    cmds = {}

    # 1. kernel trace of the benchmark (steps, transport and HVP legs; no CPU leg)
    cmds["trace"] = ["timeout", "-k", "10", "600", "rocprofv3", "--kernel-trace", "--stats", "-f", "csv", "-d",
                     f"{out}/trace", "-o", "t", "--"] + bench + ["--no-cpu-baseline"] + (
                         [] if args.kernel == "k_lse" else ["--no-hvp"])  # the counter passes' instantiation leads
    if not args.summarize_only:
        run(cmds["trace"], f"{out}/trace.log", "kernel trace")
    # 2. SQ / GRBM counters
    cmds["sq"] = ["timeout", "-s", "KILL", "180", "rocprofv3", "--pmc"] + SQ_PASS + [
        "--kernel-trace", "-f", "csv", "-d", f"{out}/sq", "-o", "s", "--"] + short_bench
    if not args.summarize_only:
        run(cmds["sq"], f"{out}/sq.log", "SQ counters")
    cmds["lds"] = ["timeout", "-s", "KILL", "180", "rocprofv3", "--pmc"] + LDS_PASS + [
        "--kernel-trace", "-f", "csv", "-d", f"{out}/lds", "-o", "l", "--"] + short_bench
    if not args.summarize_only:
        run(cmds["lds"], f"{out}/lds.log", "LDS counters")
    # 3-6. byte counters, each alone, for the workload and for a plain copy
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        cmds[ctr] = ["timeout", "-s", "KILL", "180", "rocprofv3", "--pmc", ctr, "--kernel-trace", "-f", "csv", "-d",
                     f"{out}/{ctr}", "-o", "b", "--"] + short_bench
        if not args.summarize_only:
            run(cmds[ctr], f"{out}/{ctr}.log", ctr)
        cmds["copy_" + ctr] = ["timeout", "-s", "KILL", "120", "rocprofv3", "--pmc", ctr, "--kernel-trace", "-f",
                               "csv", "-d", f"{out}/copy_{ctr}", "-o", "c", "--", py, "bench.py",
                               "--copy-calibration", "256"]
        if not args.summarize_only:
            run(cmds["copy_" + ctr], f"{out}/copy_{ctr}.log", "copy calibration " + ctr)

    # --- kernel trace ---
    stats = list(csv.DictReader(open(glob.glob(f"{out}/trace/**/t_kernel_stats.csv", recursive=True)[0])))
    lse = sorted((r for r in stats if short(r["Name"]).startswith(kname)), key=lambda r: -float(r["TotalDurationNs"]))
    if not lse:
        raise SystemExit(f"[harness] no {kname} dispatch in the trace")
    lname = short(lse[0]["Name"])
    dur_s = float(lse[0]["AverageNs"]) * 1e-9
    bench_line = None
    for line in open(f"{out}/trace.log"):
        if line.startswith("{"):
            bench_line = json.loads(line)
    src_hash = kernel_source_hash()

    # --- counters ---
    kmatch = "::" + lname + "("  # the instantiation the trace ranks first
    sq = counters(f"{out}/sq/**/s_counter_collection.csv", kmatch)
    grbm = sq.get("GRBM_GUI_ACTIVE", 0.0) / N_XCC  # summed over the XCDs
    mfma_util = 100.0 * sq.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (grbm * N_SIMD) if grbm else float("nan")
    mfma_flops = 512.0 * sq.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0)
    trans = 64.0 * sq.get("SQ_INSTS_VALU_TRANS_F32", 0.0)
    valu_per_cycle = sq.get("SQ_INSTS_VALU", 0.0) / (grbm * N_SIMD) if grbm else float("nan")
    valu_busy = 100.0 * sq.get("SQ_ACTIVE_INST_VALU", 0.0) / (N_CU * grbm) if grbm else float("nan")
    ld = counters(f"{out}/lds/**/l_counter_collection.csv", kmatch)
    grbm_l = ld.get("GRBM_GUI_ACTIVE", 0.0) / N_XCC
    lds_util = 100.0 * ld.get("SQ_LDS_IDX_ACTIVE", 0.0) / (N_CU * grbm_l) if grbm_l else float("nan")
    lds_conf = 100.0 * ld.get("SQ_LDS_BANK_CONFLICT", 0.0) / (N_CU * grbm_l) if grbm_l else float("nan")
    wave_cyc = ld.get("SQ_WAVE_CYCLES", 0.0)
    wait_lds = 100.0 * ld.get("SQ_WAIT_INST_LDS", 0.0) / wave_cyc if wave_cyc else float("nan")
    wait_any = 100.0 * ld.get("SQ_WAIT_ANY", 0.0) / wave_cyc if wave_cyc else float("nan")

    def scaled(ctr):
        # the runtime's copy kernel reads and writes 256 MiB: the counter's KiB per KiB moved
        copy_kib = counters(f"{out}/copy_{ctr}/**/c_counter_collection.csv", "copyBuffer").get(ctr, 0.0)
        scale = (256 * 1024) / copy_kib if copy_kib else float("nan")
        kib = counters(f"{out}/{ctr}/**/b_counter_collection.csv", kmatch).get(ctr, 0.0)
        return kib, copy_kib, scale, kib * scale * 1024.0

    f_kib, f_copy, f_scale, f_bytes = scaled("FETCH_SIZE")
    w_kib, w_copy, w_scale, w_bytes = scaled("WRITE_SIZE")
    hbm_bytes = f_bytes + w_bytes

    def cmdline(key):
        c = cmds[key]
        return " ".join(c[c.index("rocprofv3"):]).replace(sys.executable, "python").replace(out, args.out)

    harness_cmd = f"python -m log_domain_sinkhorn_half_amd.rocprof_harness --config {C} --out {args.out}"
    if kname != "k_lse":
        harness_cmd += f" --kernel {kname}"
    desc = DESC.get(C, f"workload {C}")

    # kernel-trace summary
    trace_md = [f"# Kernel trace on workload C{C} ({desc})", "",
                f"Made by `{harness_cmd}` (repository root); its trace pass is", "",
                f"    {cmdline('trace')}", "",
                ("the benchmark's timed Sinkhorn steps, transport leg and HVP leg.  " if kname == "k_lse" else
                 "the benchmark's timed Sinkhorn steps and transport leg.  ") + (
                    "One half-step = k_prep_keys (fp32) or" if kname == "k_lse" else
                    f"The counters cover {lname}, the P.V pass of the"),
                (f"k_prep_bias (bf16) + {lname} + k_merge (when the keys are split)." if kname == "k_lse" else
                 "transport calls (each runs after a half-step of its own)."), "",
                "| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for r in stats:
        if short(r["Name"]).startswith("k_"):
            trace_md.append(f"| {short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                            f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                            f"{float(r['Percentage']):.2f}% |")
    if bench_line:
        rf = bench_line["roofline"]
        trace_md += ["", f"The same run's bench line: {bench_line['value']} iters/s, half-step window (HIP events) "
                         f"{rf['launch_ms'] * 1e3:.1f} us against {lname} {dur_s * 1e6:.1f} us here; roofline "
                         f"{rf['bound']} {rf['achieved']} {rf['unit']} of {rf['peak']} (frac {rf['frac']})."]
    trace_md += ["", f"- kernel_source_sha256_16: {src_hash}", ""]

    # counters summary
    cnt_md = [f"# {lname} on workload C{C} ({desc}): MFMA, VALU and transcendental use", "",
              f"Made by `{harness_cmd}`; counter passes:", "", f"    {cmdline('sq')}", f"    {cmdline('lds')}", "",
              f"Means per {lname} launch; duration {dur_s * 1e6:.1f} us from the trace pass.  GRBM_GUI_ACTIVE is",
              f"summed over the {N_XCC} XCDs and divided by {N_XCC}; SIMD count {N_SIMD}.", "",
              "| quantity | value | against |", "|---|---|---|",
              f"| MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES / (GUI-active cycles x SIMDs)) | {mfma_util:.1f}% | 100% |",
              f"| executed bf16 MFMA rate (512 x SQ_INSTS_VALU_MFMA_MOPS_BF16 / duration) | "
              f"{mfma_flops / dur_s / 1e12:.1f} TFLOP/s | {PEAK_BF16 / 1e12:.1f} TFLOP/s "
              f"({mfma_flops / dur_s / PEAK_BF16:.3f}) |",
              f"| transcendental rate (64 x SQ_INSTS_VALU_TRANS_F32 / duration; all are v_exp_f32 here) | "
              f"{trans / dur_s / 1e12:.2f} T/s | {PEAK_EXP / 1e12:.2f} T/s ({trans / dur_s / PEAK_EXP:.3f}) |",
              f"| VALU instructions per SIMD cycle (SQ_INSTS_VALU / (GUI-active cycles x SIMDs)) | "
              f"{valu_per_cycle:.3f} | 1 |",
              f"| VALU busy (rocprof VALUBusy formula) | {valu_busy:.1f}% | 100% |",
              f"| MFMA instructions per launch | {sq.get('SQ_INSTS_MFMA', 0.0):.4g} | |",
              f"| waves per launch | {sq.get('SQ_WAVES', 0.0):.4g} | |",
              f"| GUI-active cycles per XCD | {grbm:.4g} | |",
              f"| LDS busy (SQ_LDS_IDX_ACTIVE / (GUI-active cycles x CUs)) | {lds_util:.1f}% | 100% |",
              f"| LDS bank-conflict cycles (same normalisation) | {lds_conf:.1f}% | 0% |",
              f"| wave time waiting for LDS instruction issue (SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES) | {wait_lds:.1f}% | |",
              f"| wave time waiting on any counter (SQ_WAIT_ANY / SQ_WAVE_CYCLES) | {wait_any:.1f}% | |",
              f"| LDS instructions per launch | {ld.get('SQ_INSTS_LDS', 0.0):.4g} | |",
              "", f"- kernel_source_sha256_16: {src_hash}", ""]

    # traffic summary (read by bench.py)
    tr_md = [f"# {lname} on workload C{C} ({desc}): HBM traffic per launch", "",
             f"Made by `{harness_cmd}`; byte passes (one counter each):", ""]
    for key in ("FETCH_SIZE", "copy_FETCH_SIZE", "WRITE_SIZE", "copy_WRITE_SIZE"):
        tr_md.append(f"    {cmdline(key)}")
    tr_md += ["", "| quantity | value |", "|---|---|",
              f"| copy calibration: FETCH_SIZE of a 256 MiB copy | {f_copy:.1f} KiB (scale x{f_scale:.3f}) |",
              f"| copy calibration: WRITE_SIZE of a 256 MiB copy | {w_copy:.1f} KiB (scale x{w_scale:.3f}) |",
              f"| {lname} FETCH_SIZE | {f_kib:.1f} KiB -> {f_bytes / 1e6:.2f} MB |",
              f"| {lname} WRITE_SIZE | {w_kib:.1f} KiB -> {w_bytes / 1e6:.2f} MB |",
              f"| HBM rate over the launch | {hbm_bytes / dur_s / 1e9:.1f} GB/s of {PEAK_HBM / 1e9:.0f} |"]
    if kname == "k_lse":
        tr_md += [f"| algorithmic bytes (clouds read once at their input precision, 20 B per point) | "
                  f"{algorithmic_bytes(C) / 1e6:.2f} MB |",
                  f"| measured / algorithmic | {hbm_bytes / algorithmic_bytes(C):.2f} |",
                  f"| operand-layout bytes (the kernel's K-slot rows read once, potential written once) | "
                  f"{operand_bytes(C) / 1e6:.2f} MB |",
                  f"| measured / operand-layout bytes | {hbm_bytes / operand_bytes(C):.2f} |", "",
                  "Traffic above the algorithmic bytes is the key operand re-read by the row blocks of a key split",
                  "(served mostly by the L2 and the MALL); at these rates HBM is far from its roof."]
    tr_md += ["",
              f"- hbm_bytes_per_launch: {int(round(hbm_bytes))}", f"- kernel_source_sha256_16: {src_hash}", ""]

    files = {"kernel_trace": trace_md, "counters": cnt_md, "traffic": tr_md}
    for kind, lines in files.items():
        text = "\n".join(lines)
        open(f"{out}/{kname}_C{C}_{kind}.md", "w").write(text)
        if args.write_profiles:
            open(os.path.join(ROOT, "profiles", f"{kname}_C{C}_{kind}.md"), "w").write(text)
    print("\n".join(cnt_md + tr_md[-8:]), flush=True)


if __name__ == "__main__":
    main()
