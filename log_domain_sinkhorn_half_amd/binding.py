"""Thin Python binding over the C ABI in include/sinkhorn.h (libsinkhorn.so).

Argument marshalling only: every step of every call runs in the HIP kernels of
libsinkhorn.so.  PyTorch provides device memory and the current HIP stream.
There is no CPU fallback: if the library is missing, every call raises.

Tensors: X [B, n, d] (or [n, d]), Y [B, m, d] (or [m, d]), float32 or bfloat16,
contiguous, on a ROCm device; a [B, n], b [B, m], f [B, n], g [B, m] float32.
Every call takes `cost` (SK_SQEUCLID or SK_COSINE); it must be the same for
all calls on one workspace.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Union

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsinkhorn.so")

SK_FP32, SK_BF16 = 0, 1
SK_SQEUCLID, SK_COSINE = 0, 1  # ground cost: ||x - y||^2, or the same between normalised points
STATUS = {0: "SK_OK", 1: "SK_EINVAL", 2: "SK_ESHAPE", 3: "SK_EDTYPE", 4: "SK_EHIP",
          5: "SK_EUNSUPPORTED", 6: "SK_EWORKSPACE"}
EXPORTS = ("sinkhorn_workspace_bytes", "sinkhorn_init_norms", "sinkhorn_half_step_f",
           "sinkhorn_half_step_g", "sinkhorn_solve", "sinkhorn_marginal_error",
           "sinkhorn_transport_workspace_bytes", "sinkhorn_barycentric_x", "sinkhorn_barycentric_y",
           "sinkhorn_apply_plan_x", "sinkhorn_apply_plan_y", "sinkhorn_hvp_workspace_bytes",
           "sinkhorn_hvp_x", "sinkhorn_hvp_y", "sinkhorn_last_error", "sinkhorn_solve_noalloc",
           "sinkhorn_range_flags")
SK_FLAG_SCORE_RANGE, SK_FLAG_NONFINITE = 1, 2  # bits of the workspace's status word
SK_NOALLOC_MAX_BYTES = 64 * 1024 * 1024  # built-in scratch array of sinkhorn_solve_noalloc


class SkProblem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("n", ctypes.c_int64), ("m", ctypes.c_int64),
                ("d", ctypes.c_int64), ("dtype", ctypes.c_int32), ("cost", ctypes.c_int32)]


class SinkhornError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def load_library(path: Optional[str] = None):
    """Load libsinkhorn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m log_domain_sinkhorn_half_amd.build` "
                           "(there is no CPU fallback)")
    lib = ctypes.CDLL(p)
    vp, sz, f32p = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p
    P = ctypes.POINTER(SkProblem)
    lib.sinkhorn_workspace_bytes.argtypes = [P]
    lib.sinkhorn_workspace_bytes.restype = sz
    lib.sinkhorn_init_norms.argtypes = [P, vp, vp, f32p, f32p, vp, sz, vp]
    lib.sinkhorn_init_norms.restype = ctypes.c_int
    lib.sinkhorn_half_step_f.argtypes = [P, vp, vp, vp, sz, f32p, ctypes.c_float, f32p, vp]
    lib.sinkhorn_half_step_f.restype = ctypes.c_int
    lib.sinkhorn_half_step_g.argtypes = [P, vp, vp, vp, sz, f32p, ctypes.c_float, f32p, vp]
    lib.sinkhorn_half_step_g.restype = ctypes.c_int
    lib.sinkhorn_solve.argtypes = [P, vp, vp, f32p, f32p, ctypes.POINTER(ctypes.c_float), ctypes.c_int64,
                                   ctypes.c_int64, f32p, f32p, vp, sz, vp]
    lib.sinkhorn_solve.restype = ctypes.c_int
    lib.sinkhorn_marginal_error.argtypes = [P, vp, vp, vp, sz, f32p, f32p, ctypes.c_float, f32p, vp]
    lib.sinkhorn_marginal_error.restype = ctypes.c_int
    lib.sinkhorn_transport_workspace_bytes.argtypes = [P]
    lib.sinkhorn_transport_workspace_bytes.restype = sz
    for name in ("sinkhorn_barycentric_x", "sinkhorn_barycentric_y"):
        fn = getattr(lib, name)
        fn.argtypes = [P, vp, vp, vp, sz, f32p, f32p, ctypes.c_float, f32p, f32p, vp]
        fn.restype = ctypes.c_int
    for name in ("sinkhorn_apply_plan_x", "sinkhorn_apply_plan_y"):
        fn = getattr(lib, name)
        fn.argtypes = [P, vp, vp, vp, sz, f32p, f32p, ctypes.c_float, f32p, ctypes.c_int64, f32p, vp]
        fn.restype = ctypes.c_int
    lib.sinkhorn_hvp_workspace_bytes.argtypes = [P]
    lib.sinkhorn_hvp_workspace_bytes.restype = sz
    for name in ("sinkhorn_hvp_x", "sinkhorn_hvp_y"):
        fn = getattr(lib, name)
        fn.argtypes = [P, vp, vp, vp, sz, f32p, f32p, ctypes.c_float, f32p, ctypes.c_int64, ctypes.c_float,
                       f32p, vp]
        fn.restype = ctypes.c_int
    lib.sinkhorn_solve_noalloc.argtypes = [P, vp, vp, f32p, f32p, ctypes.POINTER(ctypes.c_float), ctypes.c_int64,
                                           ctypes.c_int64, f32p, f32p, vp, vp]
    lib.sinkhorn_solve_noalloc.restype = ctypes.c_int
    lib.sinkhorn_range_flags.argtypes = [P, vp, sz, vp, vp]
    lib.sinkhorn_range_flags.restype = ctypes.c_int
    lib.sinkhorn_last_error.argtypes = []
    lib.sinkhorn_last_error.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        msg = load_library().sinkhorn_last_error().decode(errors="replace")
        raise SinkhornError(status, msg)


def _call(name: str, *args) -> None:
    """Call one entry point of the library; the arguments (and so every check
    made while marshalling them) are evaluated before the library is loaded."""
    _check(getattr(load_library(), name)(*args))


def _as3(t: torch.Tensor) -> torch.Tensor:
    return t if t.dim() == 3 else t.unsqueeze(0)


def _as2(t: torch.Tensor) -> torch.Tensor:
    return t if t.dim() == 2 else t.unsqueeze(0)


def problem_of(X: torch.Tensor, Y: torch.Tensor, cost: int = SK_SQEUCLID) -> SkProblem:
    X3, Y3 = _as3(X), _as3(Y)
    if X3.dim() != 3 or Y3.dim() != 3 or X3.shape[0] != Y3.shape[0] or X3.shape[2] != Y3.shape[2]:
        raise ValueError(f"X {tuple(X.shape)} and Y {tuple(Y.shape)} must be [B,n,d] and [B,m,d]")
    if X.dtype != Y.dtype or X.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("X and Y must both be float32 or both bfloat16")
    dt = SK_FP32 if X.dtype == torch.float32 else SK_BF16
    return SkProblem(X3.shape[0], X3.shape[1], Y3.shape[1], X3.shape[2], dt, int(cost))


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}")
    return t.data_ptr()


def _shape(t: Optional[torch.Tensor], name: str, shape) -> None:
    """Raise ValueError unless t has `shape` ([B, ...]; a single problem may also
    drop the leading 1).  The kernels index every array by (batch, n, m, d, c),
    so a wrongly sized tensor would be read or written out of bounds."""
    if t is None:
        return
    got = tuple(t.shape)
    want = tuple(int(v) for v in shape)
    if got != want and not (want[0] == 1 and got == want[1:]):
        raise ValueError(f"{name} has shape {got}, expected {want}")


def _same_device(X: torch.Tensor, *named) -> None:
    for name, t in named:
        if t is not None and t.device != X.device:
            raise ValueError(f"{name} is on {t.device}, but X is on {X.device}")


def _stream(X: torch.Tensor) -> int:
    """The current HIP stream of X's device (the library launches there)."""
    return torch.cuda.current_stream(X.device).cuda_stream


def workspace_bytes(batch: int, n: int, m: int, d: int, dtype: int = SK_FP32, cost: int = SK_SQEUCLID) -> int:
    p = SkProblem(batch, n, m, d, dtype, cost)
    nb = load_library().sinkhorn_workspace_bytes(ctypes.byref(p))
    if nb == 0:
        _check(1)
    return int(nb)


def alloc_workspace(X: torch.Tensor, Y: torch.Tensor, transport: bool = False, cost: int = SK_SQEUCLID,
                    hvp: bool = False) -> torch.Tensor:
    """Device workspace for the solver (transport=True: also for the barycentric and
    plan-application calls; hvp=True: also for the Hessian-vector products)."""
    p = problem_of(X, Y, cost)
    lib = load_library()
    size_fn = (lib.sinkhorn_hvp_workspace_bytes if hvp else
               lib.sinkhorn_transport_workspace_bytes if transport else lib.sinkhorn_workspace_bytes)
    nb = size_fn(ctypes.byref(p))
    if nb == 0:
        _check(1)
    return torch.empty(nb, dtype=torch.uint8, device=X.device)


def init_norms(X, Y, a, b, ws, cost: int = SK_SQEUCLID):
    p = problem_of(X, Y, cost)
    _shape(a, "a", (p.batch, p.n))
    _shape(b, "b", (p.batch, p.m))
    _same_device(X, ("Y", Y), ("a", a), ("b", b), ("ws", ws))
    _call("sinkhorn_init_norms",
        ctypes.byref(p), _dev(X, "X"), _dev(Y, "Y"), _dev(a, "a", torch.float32),
        _dev(b, "b", torch.float32), _dev(ws, "ws"), ws.numel() * ws.element_size(), _stream(X))


def half_step_f(X, Y, ws, g, eps: float, f: Optional[torch.Tensor] = None, cost: int = SK_SQEUCLID) -> torch.Tensor:
    p = problem_of(X, Y, cost)
    _shape(g, "g", (p.batch, p.m))
    _shape(f, "f", (p.batch, p.n))
    _same_device(X, ("Y", Y), ("ws", ws), ("g", g), ("f", f))
    if f is None:
        f = torch.empty((p.batch, p.n), dtype=torch.float32, device=X.device)
    _call("sinkhorn_half_step_f",
        ctypes.byref(p), _dev(X, "X"), _dev(Y, "Y"), _dev(ws, "ws"), ws.numel() * ws.element_size(),
        _dev(g, "g", torch.float32), float(eps), _dev(f, "f", torch.float32), _stream(X))
    return f


def half_step_g(X, Y, ws, f, eps: float, g: Optional[torch.Tensor] = None, cost: int = SK_SQEUCLID) -> torch.Tensor:
    p = problem_of(X, Y, cost)
    _shape(f, "f", (p.batch, p.n))
    _shape(g, "g", (p.batch, p.m))
    _same_device(X, ("Y", Y), ("ws", ws), ("f", f), ("g", g))
    if g is None:
        g = torch.empty((p.batch, p.m), dtype=torch.float32, device=X.device)
    _call("sinkhorn_half_step_g",
        ctypes.byref(p), _dev(X, "X"), _dev(Y, "Y"), _dev(ws, "ws"), ws.numel() * ws.element_size(),
        _dev(f, "f", torch.float32), float(eps), _dev(g, "g", torch.float32), _stream(X))
    return g


def solve(X, Y, a, b, eps: Union[float, Sequence[float]], iters: int, f=None, g=None, ws=None,
          cost: int = SK_SQEUCLID):
    """Run sinkhorn_solve; f and g are in/out (zeros if not given).  Returns (f, g)."""
    p = problem_of(X, Y, cost)
    for name, t, shp in (("a", a, (p.batch, p.n)), ("b", b, (p.batch, p.m)), ("f", f, (p.batch, p.n)),
                         ("g", g, (p.batch, p.m))):
        _shape(t, name, shp)
    _same_device(X, ("Y", Y), ("a", a), ("b", b), ("f", f), ("g", g), ("ws", ws))
    if f is None:
        f = torch.zeros((p.batch, p.n), dtype=torch.float32, device=X.device)
    if g is None:
        g = torch.zeros((p.batch, p.m), dtype=torch.float32, device=X.device)
    if ws is None:
        ws = alloc_workspace(X, Y, cost=cost)
    e = [float(eps)] if isinstance(eps, (int, float)) else [float(v) for v in eps]
    earr = (ctypes.c_float * len(e))(*e)
    _call("sinkhorn_solve",
        ctypes.byref(p), _dev(X, "X"), _dev(Y, "Y"), _dev(a, "a", torch.float32), _dev(b, "b", torch.float32),
        earr, len(e), int(iters), _dev(f, "f", torch.float32), _dev(g, "g", torch.float32), _dev(ws, "ws"),
        ws.numel() * ws.element_size(), _stream(X))
    return f, g


def solve_noalloc(X, Y, a, b, eps: Union[float, Sequence[float]], iters: int, f=None, g=None,
                  flags: Optional[torch.Tensor] = None, cost: int = SK_SQEUCLID):
    """sinkhorn_solve_noalloc: the solve on the library's built-in scratch array (no
    workspace; problems up to SK_NOALLOC_MAX_BYTES of workspace).  f and g are in/out
    (zeros if not given); flags, if given, is a device int32 [1] that receives the
    status word.  Returns (f, g)."""
    p = problem_of(X, Y, cost)
    for name, t, shp in (("a", a, (p.batch, p.n)), ("b", b, (p.batch, p.m)), ("f", f, (p.batch, p.n)),
                         ("g", g, (p.batch, p.m)), ("flags", flags, (1,))):
        _shape(t, name, shp)
    _same_device(X, ("Y", Y), ("a", a), ("b", b), ("f", f), ("g", g), ("flags", flags))
    if f is None:
        f = torch.zeros((p.batch, p.n), dtype=torch.float32, device=X.device)
    if g is None:
        g = torch.zeros((p.batch, p.m), dtype=torch.float32, device=X.device)
    e = [float(eps)] if isinstance(eps, (int, float)) else [float(v) for v in eps]
    earr = (ctypes.c_float * len(e))(*e)
    _call("sinkhorn_solve_noalloc",
          ctypes.byref(p), _dev(X, "X"), _dev(Y, "Y"), _dev(a, "a", torch.float32), _dev(b, "b", torch.float32),
          earr, len(e), int(iters), _dev(f, "f", torch.float32), _dev(g, "g", torch.float32),
          None if flags is None else _dev(flags, "flags", torch.int32), _stream(X))
    return f, g


def range_flags(X, Y, ws, cost: int = SK_SQEUCLID) -> int:
    """Status word of ws (SK_FLAG_* bits set since the last init_norms); synchronises
    the current stream to read it."""
    p = problem_of(X, Y, cost)
    _same_device(X, ("ws", ws))
    out = torch.zeros(1, dtype=torch.int32, device=X.device)
    _call("sinkhorn_range_flags", ctypes.byref(p), _dev(ws, "ws"), ws.numel() * ws.element_size(),
          _dev(out, "flags", torch.int32), _stream(X))
    return int(out.item())


def marginal_error(X, Y, ws, f, g, eps: float, err: Optional[torch.Tensor] = None,
                   cost: int = SK_SQEUCLID) -> torch.Tensor:
    p = problem_of(X, Y, cost)
    _shape(f, "f", (p.batch, p.n))
    _shape(g, "g", (p.batch, p.m))
    _shape(err, "err", (p.batch, 2))
    _same_device(X, ("Y", Y), ("ws", ws), ("f", f), ("g", g), ("err", err))
    if err is None:
        err = torch.empty((p.batch, 2), dtype=torch.float32, device=X.device)
    _call("sinkhorn_marginal_error",
        ctypes.byref(p), _dev(X, "X"), _dev(Y, "Y"), _dev(ws, "ws"), ws.numel() * ws.element_size(),
        _dev(f, "f", torch.float32), _dev(g, "g", torch.float32), float(eps), _dev(err, "err", torch.float32),
        _stream(X))
    return err


def _barycentric(name, X, Y, ws, f, g, eps, rows, bary, grad, with_grad, cost):
    p = problem_of(X, Y, cost)
    shape = (p.batch, rows(p), p.d)
    _shape(f, "f", (p.batch, p.n))
    _shape(g, "g", (p.batch, p.m))
    _shape(bary, "bary", shape)
    _shape(grad, "grad", shape)
    _same_device(X, ("Y", Y), ("ws", ws), ("f", f), ("g", g), ("bary", bary), ("grad", grad))
    if bary is None:
        bary = torch.empty(shape, dtype=torch.float32, device=X.device)
    if grad is None and with_grad:
        grad = torch.empty(shape, dtype=torch.float32, device=X.device)
    _call(name,
        ctypes.byref(p), _dev(X, "X"), _dev(Y, "Y"), _dev(ws, "ws"), ws.numel() * ws.element_size(),
        _dev(f, "f", torch.float32), _dev(g, "g", torch.float32), float(eps), _dev(bary, "bary", torch.float32),
        None if grad is None else _dev(grad, "grad", torch.float32), _stream(X))
    return bary, grad


def barycentric_x(X, Y, ws, f, g, eps: float, bary=None, grad=None, with_grad: bool = True,
                  cost: int = SK_SQEUCLID):
    """Barycentric projection of the points of X under the plan of (f, g), and the
    gradient sum_j P_ij 2 (x_i - y_j).  ws must come from alloc_workspace(..., transport=True)."""
    return _barycentric("sinkhorn_barycentric_x", X, Y, ws, f, g, eps, lambda p: p.n, bary, grad, with_grad, cost)


def barycentric_y(X, Y, ws, f, g, eps: float, bary=None, grad=None, with_grad: bool = True,
                  cost: int = SK_SQEUCLID):
    """Barycentric projection of the points of Y (columns of the plan) and the
    gradient sum_i P_ij 2 (y_j - x_i)."""
    return _barycentric("sinkhorn_barycentric_y", X, Y, ws, f, g, eps, lambda p: p.m, bary, grad, with_grad, cost)


def _apply(name, X, Y, ws, f, g, eps, M, keys, rows, out, cost):
    p = problem_of(X, Y, cost)
    squeeze = M.dim() == 2
    M3 = M.unsqueeze(-1) if squeeze else M
    c = M3.shape[-1]
    _shape(f, "f", (p.batch, p.n))
    _shape(g, "g", (p.batch, p.m))
    _shape(M3, "matrix", (p.batch, keys(p), c))
    _shape(out, "out", (p.batch, rows(p), c) if not squeeze else (p.batch, rows(p)))
    _same_device(X, ("Y", Y), ("ws", ws), ("f", f), ("g", g), ("matrix", M), ("out", out))
    if out is not None and squeeze:
        out = out.reshape(p.batch, rows(p), 1)
    if out is None:
        out = torch.empty((p.batch, rows(p), c), dtype=torch.float32, device=X.device)
    _call(name,
        ctypes.byref(p), _dev(X, "X"), _dev(Y, "Y"), _dev(ws, "ws"), ws.numel() * ws.element_size(),
        _dev(f, "f", torch.float32), _dev(g, "g", torch.float32), float(eps), _dev(M3, "matrix", torch.float32),
        int(c), _dev(out, "out", torch.float32), _stream(X))
    return out.squeeze(-1) if squeeze else out


def apply_plan_x(X, Y, ws, f, g, eps: float, V, out=None, cost: int = SK_SQEUCLID):
    """(P V)_i = sum_j P_ij V_j for V [B, m, c] (or [B, m]); ws from alloc_workspace(..., transport=True)."""
    return _apply("sinkhorn_apply_plan_x", X, Y, ws, f, g, eps, V, lambda p: p.m, lambda p: p.n, out, cost)


def apply_plan_y(X, Y, ws, f, g, eps: float, U, out=None, cost: int = SK_SQEUCLID):
    """(P^T U)_j = sum_i P_ij U_i for U [B, n, c] (or [B, n])."""
    return _apply("sinkhorn_apply_plan_y", X, Y, ws, f, g, eps, U, lambda p: p.n, lambda p: p.m, out, cost)


def _hvp(name, X, Y, ws, f, g, eps, V, cg_iters, cg_tol, out, rows):
    p = problem_of(X, Y)
    _shape(f, "f", (p.batch, p.n))
    _shape(g, "g", (p.batch, p.m))
    _shape(V, "V", (p.batch, rows(p), p.d))
    _shape(out, "out", (p.batch, rows(p), p.d))
    _same_device(X, ("Y", Y), ("ws", ws), ("f", f), ("g", g), ("V", V), ("out", out))
    if out is None:
        out = torch.empty_like(V, dtype=torch.float32)
    _call(name,
        ctypes.byref(p), _dev(X, "X"), _dev(Y, "Y"), _dev(ws, "ws"), ws.numel() * ws.element_size(),
        _dev(f, "f", torch.float32), _dev(g, "g", torch.float32), float(eps), _dev(V, "V", torch.float32),
        int(cg_iters), float(cg_tol), _dev(out, "out", torch.float32), _stream(X))
    return out


def hvp_x(X, Y, ws, f, g, eps: float, V, cg_iters: int = 200, cg_tol: float = 1e-6, out=None):
    """Hessian of the entropic OT value in X applied to V [B, n, d], at optimal (f, g).
    ws from alloc_workspace(..., hvp=True)."""
    return _hvp("sinkhorn_hvp_x", X, Y, ws, f, g, eps, V, cg_iters, cg_tol, out, lambda p: p.n)


def hvp_y(X, Y, ws, f, g, eps: float, V, cg_iters: int = 200, cg_tol: float = 1e-6, out=None):
    """Hessian of the entropic OT value in Y applied to V [B, m, d], at optimal (f, g)."""
    return _hvp("sinkhorn_hvp_y", X, Y, ws, f, g, eps, V, cg_iters, cg_tol, out, lambda p: p.m)
