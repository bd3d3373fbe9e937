"""Host-only checks of the C ABI library (no GPU needed).

The library must load, export every function declared in include/sinkhorn.h,
size its workspace linearly in (n+m)*d, and reject invalid arguments on the
host before anything touches a device.
"""

import ctypes
import os
import re
import subprocess

import pytest

from log_domain_sinkhorn_half_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sinkhorn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sinkhorn_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libsinkhorn.so is not built (run __graft_entry__.build())")
    return binding.load_library()


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ("sinkhorn_init_norms", "sinkhorn_half_step_f", "sinkhorn_half_step_g", "sinkhorn_solve",
              "sinkhorn_marginal_error", "sinkhorn_workspace_bytes", "sinkhorn_last_error",
              "sinkhorn_transport_workspace_bytes", "sinkhorn_barycentric_x", "sinkhorn_barycentric_y"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (sinkhorn_\w+)", out))
    for n in _declared_functions():
        assert n in exported, n
        assert hasattr(lib, n)
    assert set(binding.EXPORTS) <= exported


def test_library_has_gfx950_code_object():
    # the offload bundle embedded by hipcc names its target
    data = open(binding.LIB_PATH, "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in data


def _prob(batch=1, n=10, m=12, d=3, dtype=0):
    return binding.SkProblem(batch, n, m, d, dtype)


def test_workspace_is_linear_not_quadratic(lib):
    small = lib.sinkhorn_workspace_bytes(ctypes.byref(_prob(1, 70000, 70000, 3)))
    big = lib.sinkhorn_workspace_bytes(ctypes.byref(_prob(1, 140000, 140000, 3)))
    assert 0 < small < 200 * 2 ** 20
    assert big < 2.2 * small  # O((n+m)d), never O(nm)
    assert lib.sinkhorn_workspace_bytes(ctypes.byref(_prob(1, 65536, 32768, 128, 1))) > 0
    assert lib.sinkhorn_workspace_bytes(ctypes.byref(_prob(1, 100, 100, 88, 0))) > 0


@pytest.mark.parametrize("p,status", [
    (None, 1),
    (_prob(n=0), 2),
    (_prob(m=-3), 2),
    (_prob(batch=0), 2),
    (_prob(d=0), 2),
    (_prob(d=2000), 5),
    (_prob(d=1025), 5),
    (_prob(d=1025, dtype=1), 5),
    (_prob(dtype=7), 3),
])
def test_invalid_problem_rejected_before_launch(lib, p, status):
    ptr = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    arg = ctypes.byref(p) if p is not None else None
    st = lib.sinkhorn_half_step_f(arg, ptr, ptr, ptr, 1 << 40, ptr, 0.1, ptr, None)
    assert st == status
    assert lib.sinkhorn_last_error()
    if p is not None:
        assert lib.sinkhorn_workspace_bytes(arg) == 0


def test_other_argument_errors(lib):
    p = _prob()
    need = lib.sinkhorn_workspace_bytes(ctypes.byref(p))
    ptr = ctypes.c_void_p(0x1000)
    bp = ctypes.byref(p)
    # workspace too small / missing
    assert lib.sinkhorn_half_step_f(bp, ptr, ptr, ptr, need - 1, ptr, 0.1, ptr, None) == 6
    assert lib.sinkhorn_half_step_g(bp, ptr, ptr, None, need, ptr, 0.1, ptr, None) == 6
    # NULL data pointers
    assert lib.sinkhorn_half_step_f(bp, None, ptr, ptr, need, ptr, 0.1, ptr, None) == 1
    assert lib.sinkhorn_init_norms(bp, ptr, ptr, None, ptr, ptr, need, None) == 1
    # bad eps
    for e in (0.0, -1.0, float("inf"), float("nan")):
        assert lib.sinkhorn_half_step_f(bp, ptr, ptr, ptr, need, ptr, e, ptr, None) == 1
        assert lib.sinkhorn_marginal_error(bp, ptr, ptr, ptr, need, ptr, ptr, e, ptr, None) == 1
    # solve: iters < 0, wrong n_eps, bad schedule entry
    E = (ctypes.c_float * 3)(0.1, 0.2, 0.3)
    assert lib.sinkhorn_solve(bp, ptr, ptr, ptr, ptr, E, 1, -1, ptr, ptr, ptr, need, None) == 1
    assert lib.sinkhorn_solve(bp, ptr, ptr, ptr, ptr, E, 2, 3, ptr, ptr, ptr, need, None) == 1
    assert lib.sinkhorn_solve(bp, ptr, ptr, ptr, ptr, None, 1, 3, ptr, ptr, ptr, need, None) == 1
    Ebad = (ctypes.c_float * 3)(0.1, 0.0, 0.3)
    assert lib.sinkhorn_solve(bp, ptr, ptr, ptr, ptr, Ebad, 3, 3, ptr, ptr, ptr, need, None) == 1
    assert b"eps[1]" in lib.sinkhorn_last_error()


def test_transport_workspace_and_argument_errors(lib):
    p = _prob(1, 700, 500, 3)
    bp = ctypes.byref(p)
    base = lib.sinkhorn_workspace_bytes(bp)
    full = lib.sinkhorn_transport_workspace_bytes(bp)
    assert full > base > 0
    # linear in (n+m)d and bounded at the large workloads
    assert lib.sinkhorn_transport_workspace_bytes(ctypes.byref(_prob(1, 65536, 32768, 128, 1))) < 2 ** 30
    assert lib.sinkhorn_transport_workspace_bytes(ctypes.byref(_prob(1, 100, 100, 88, 0))) > 0
    assert lib.sinkhorn_transport_workspace_bytes(ctypes.byref(_prob(d=1025))) == 0
    ptr = ctypes.c_void_p(0x1000)
    for fn in (lib.sinkhorn_barycentric_x, lib.sinkhorn_barycentric_y):
        # the solver-sized workspace is too small for the transport calls
        assert fn(bp, ptr, ptr, ptr, base, ptr, ptr, 0.1, ptr, None, None) == 6
        assert b"sinkhorn_transport_workspace_bytes" in lib.sinkhorn_last_error()
        # bary is required, grad is optional (NULL passes validation up to the launch)
        assert fn(bp, ptr, ptr, ptr, full, ptr, ptr, 0.1, None, ptr, None) == 1
        assert fn(bp, ptr, ptr, ptr, full, None, ptr, 0.1, ptr, ptr, None) == 1
        assert fn(bp, ptr, ptr, ptr, full, ptr, ptr, 0.0, ptr, ptr, None) == 1
        # wide problems (fp32 past d = 88, bf16 past d = 256) take the weights-buffer
        # passes: their transport workspace holds it, and a smaller one is refused
        for wide in (_prob(1, 300, 200, 89, 0), _prob(1, 300, 200, 300, 1), _prob(1, 300, 200, 1024, 0)):
            wb = lib.sinkhorn_transport_workspace_bytes(ctypes.byref(wide))
            assert wb > lib.sinkhorn_workspace_bytes(ctypes.byref(wide)) > 0
            assert fn(ctypes.byref(wide), ptr, ptr, ptr, wb - 256, ptr, ptr, 0.1, ptr, ptr, None) == 6


def test_cost_field_validation(lib):
    ptr = ctypes.c_void_p(0x1000)
    bad = binding.SkProblem(1, 10, 12, 3, 0, 7)
    assert lib.sinkhorn_workspace_bytes(ctypes.byref(bad)) == 0
    assert lib.sinkhorn_half_step_f(ctypes.byref(bad), ptr, ptr, ptr, 1 << 40, ptr, 0.1, ptr, None) == 1
    assert b"cost" in lib.sinkhorn_last_error()
    # the cosine cost uses the split layout: bf16 inputs are limited like fp32 ones
    assert lib.sinkhorn_workspace_bytes(ctypes.byref(binding.SkProblem(1, 10, 12, 100, 1, 1))) == 0
    assert lib.sinkhorn_workspace_bytes(ctypes.byref(binding.SkProblem(1, 10, 12, 100, 1, 0))) > 0
    sq = lib.sinkhorn_workspace_bytes(ctypes.byref(binding.SkProblem(1, 1000, 1000, 64, 1, 0)))
    cos = lib.sinkhorn_workspace_bytes(ctypes.byref(binding.SkProblem(1, 1000, 1000, 64, 1, 1)))
    assert cos > sq > 0
    text = open(HEADER).read()
    assert "SK_COST_SQEUCLID = 0" in text and "SK_COST_COSINE = 1" in text


def test_plan_and_hvp_entry_points_validate(lib):
    p = _prob(1, 300, 200, 3)
    bp = ctypes.byref(p)
    t = lib.sinkhorn_transport_workspace_bytes(bp)
    h = lib.sinkhorn_hvp_workspace_bytes(bp)
    assert h > t > lib.sinkhorn_workspace_bytes(bp) > 0
    assert lib.sinkhorn_hvp_workspace_bytes(ctypes.byref(_prob(1, 65536, 32768, 128, 1))) < 2 ** 31
    ptr = ctypes.c_void_p(0x1000)
    for fn in (lib.sinkhorn_apply_plan_x, lib.sinkhorn_apply_plan_y):
        assert fn(bp, ptr, ptr, ptr, t - 1, ptr, ptr, 0.1, ptr, 3, ptr, None) == 6
        assert fn(bp, ptr, ptr, ptr, t, ptr, ptr, 0.1, ptr, 0, ptr, None) == 1       # no columns
        assert fn(bp, ptr, ptr, ptr, t, ptr, ptr, 0.1, None, 3, ptr, None) == 1      # no matrix
        assert fn(bp, ptr, ptr, ptr, t, ptr, ptr, -1.0, ptr, 3, ptr, None) == 1
    for fn in (lib.sinkhorn_hvp_x, lib.sinkhorn_hvp_y):
        assert fn(bp, ptr, ptr, ptr, t, ptr, ptr, 0.1, ptr, 10, 1e-6, ptr, None) == 6  # transport size is too small
        assert b"sinkhorn_hvp_workspace_bytes" in lib.sinkhorn_last_error()
        assert fn(bp, ptr, ptr, ptr, h, ptr, ptr, 0.1, ptr, -1, 1e-6, ptr, None) == 1
        assert fn(bp, ptr, ptr, ptr, h, ptr, ptr, 0.1, ptr, 10, float("nan"), ptr, None) == 1
        assert fn(bp, ptr, ptr, ptr, h, ptr, ptr, 0.1, None, 10, 1e-6, ptr, None) == 1
        cos = binding.SkProblem(1, 300, 200, 3, 0, 1)
        hc = lib.sinkhorn_hvp_workspace_bytes(ctypes.byref(cos))
        assert fn(ctypes.byref(cos), ptr, ptr, ptr, hc, ptr, ptr, 0.1, ptr, 10, 1e-6, ptr, None) == 5


def test_missing_library_fails_loudly(tmp_path):
    """No CPU fallback: a library path that does not exist raises, naming the build step."""
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        binding.load_library(str(tmp_path / "libsinkhorn.so"))


def test_range_flags_query_validates(lib):
    p = _prob(1, 300, 200, 3)
    bp = ctypes.byref(p)
    need = lib.sinkhorn_workspace_bytes(bp)
    ptr = ctypes.c_void_p(0x1000)
    assert lib.sinkhorn_range_flags(bp, ptr, need - 1, ptr, None) == 6
    assert lib.sinkhorn_range_flags(bp, None, need, ptr, None) == 6
    assert lib.sinkhorn_range_flags(bp, ptr, need, None, None) == 1
    assert lib.sinkhorn_range_flags(None, ptr, need, ptr, None) == 1
    text = open(HEADER).read()
    assert "#define SK_FLAG_SCORE_RANGE 1u" in text and "#define SK_FLAG_NONFINITE 2u" in text
    assert binding.SK_FLAG_SCORE_RANGE == 1 and binding.SK_FLAG_NONFINITE == 2
