"""MI355X-native log-domain Sinkhorn half-steps (squared-Euclidean or cosine cost).

The compute lives in libsinkhorn.so (HIP, gfx950), declared in include/sinkhorn.h;
``binding`` marshals torch tensors into that C ABI.  ``inputs`` holds the seeded
synthetic workloads.
"""

from .binding import (SK_BF16, SK_COSINE, SK_FP32, SK_SQEUCLID, SinkhornError, alloc_workspace, apply_plan_x,
                      apply_plan_y, barycentric_x, barycentric_y, half_step_f, half_step_g, hvp_x, hvp_y,
                      init_norms, load_library, marginal_error, problem_of, range_flags, solve, solve_noalloc,
                      workspace_bytes)

__all__ = ["SK_BF16", "SK_COSINE", "SK_FP32", "SK_SQEUCLID", "SinkhornError", "alloc_workspace", "apply_plan_x",
           "apply_plan_y", "barycentric_x", "barycentric_y", "half_step_f", "half_step_g", "hvp_x", "hvp_y",
           "init_norms", "load_library", "marginal_error", "problem_of", "range_flags", "solve", "solve_noalloc",
           "workspace_bytes"]
