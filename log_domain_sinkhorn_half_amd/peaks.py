"""Peak-rate microbenchmarks (csrc/peaks.hip): the exp and MFMA denominators.

    python -m log_domain_sinkhorn_half_amd.peaks

prints one JSON line with the measured v_exp_f32 rate (exps/s), the dense
bf16 and fp32 MFMA rates (flop/s) of GPU 0, and the exp rate when every exp
also carries an add (fp32 half-step) or an FMA and an add (bf16 half-step),
and the bf16 MFMA rate of the d = 128 half-step's tile structure with no memory
traffic (MFMA chains whose results feed the exps, a barrier every 4 tiles), next to the figures the roofline
uses (256 CUs x 4 SIMDs x 8 transcendental lanes x 2.4 GHz; AMD's dense
2516.6 and 157.3 TFLOP/s).  The benchmark prices against the larger of the
spec and the measurement, so a weak measurement cannot inflate a fraction.
"""

from __future__ import annotations

import ctypes
import json
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libskpeaks.so")

SPEC = {"exp": 256 * 4 * 8 * 2.4e9, "bf16": 2516.6e12, "fp32": 157.3e12}
KERNELS = {"exp": (0, 20000), "bf16": (1, 8000), "fp32": (2, 4000)}  # (which, loop trips)
# exps with the half-steps' other VALU work per score, against the same exp figure
MIXES = {"exp+add": (3, 20000), "fma+exp+add": (4, 20000)}
# the bf16 half-step's key-tile structure (d = 128) without memory traffic, against the bf16 figure,
# at 2 waves per SIMD (512 workgroups of 4 waves)
TILE = {"tile": (5, 2000)}
BLOCKS = {"tile": 512}


def measure(name: str, blocks: int = 256 * 8) -> dict:
    """Rate of one microbenchmark on the current device (best of three launches)."""
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m log_domain_sinkhorn_half_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    lib.sk_peak.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_float),
                            ctypes.POINTER(ctypes.c_double)]
    lib.sk_peak.restype = ctypes.c_int
    which, iters = KERNELS.get(name) or MIXES.get(name) or TILE[name]
    blocks = BLOCKS.get(name, blocks)
    best = None
    for _ in range(3):
        ms, ops = ctypes.c_float(0.0), ctypes.c_double(0.0)
        rc = lib.sk_peak(which, blocks, iters, ctypes.byref(ms), ctypes.byref(ops))
        if rc != 0:
            raise RuntimeError(f"sk_peak({name}) failed with HIP error {rc}")
        rate = ops.value / (ms.value / 1e3)
        best = rate if best is None else max(best, rate)
    spec = SPEC[name] if name in SPEC else (SPEC["bf16"] if name in TILE else SPEC["exp"])
    return {"measured": best, "spec": spec, "ratio": best / spec}


def main():
    out = {name: measure(name) for name in list(KERNELS) + list(MIXES) + list(TILE)}
    print(json.dumps({k: {kk: (round(vv, 4) if kk == "ratio" else float(f"{vv:.4g}")) for kk, vv in v.items()}
                      for k, v in out.items()}), flush=True)


if __name__ == "__main__":
    main()
