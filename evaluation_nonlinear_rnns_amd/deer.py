"""Python binding of libdeer (include/deer.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of the solver runs in the library's HIP kernels.  The
functions keep the C names.  Loading fails loudly when the library has not
been built (``python -m evaluation_nonlinear_rnns_amd.build``) -- there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdeer.so")

DEER_MODE_DENSE = 0
DEER_MODE_DIAG = 1
DEER_MODE_JACOBI = 2
DEER_MODE_PICARD = 3
DEER_CELL_TANH = 0
DEER_CELL_GRU = 1
MODES = {"dense": DEER_MODE_DENSE, "diag": DEER_MODE_DIAG, "jacobi": DEER_MODE_JACOBI, "picard": DEER_MODE_PICARD}
CELLS = {"tanh": DEER_CELL_TANH, "gru": DEER_CELL_GRU}

DEER_OK = 0
DEER_NOT_CONVERGED = 1
SEQ_CONVERGED, SEQ_NOT_CONVERGED, SEQ_NONFINITE, SEQ_STALLED = 0, 1, 2, 3
ERRORS = {-1: "DEER_ERR_INVALID", -2: "DEER_ERR_UNSUPPORTED", -3: "DEER_ERR_WORKSPACE",
          -4: "DEER_ERR_HIP", -5: "DEER_ERR_DEVICE"}

# Every symbol include/deer.h declares.
EXPORTS = ("deer_workspace_size", "deer_workspace_init", "deer_solve", "linear_scan_workspace_size",
           "linear_scan_diag", "linear_scan_diag_noalloc", "linear_scan_dense", "deer_rollout_workspace_size",
           "deer_rollout", "deer_lle_workspace_size", "deer_lle",
           "deer_broyden_workspace_size", "deer_solve_broyden", "linear_scan_dplr_workspace_size",
           "linear_scan_dplr", "deer_profile_enable", "deer_profile_read", "deer_bandwidth_probe", "deer_last_error")


class DeerError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code


class BroydenOpts(ctypes.Structure):
    _fields_ = [("rank", ctypes.c_int), ("multisecant", ctypes.c_int), ("alpha", ctypes.c_float),
                ("damping", ctypes.c_float), ("gram_reg", ctypes.c_float), ("chunk", ctypes.c_int),
                ("sketch", ctypes.c_void_p), ("stall_window", ctypes.c_int)]


class SolveOpts(ctypes.Structure):
    """deer_solve_opts_t; the defaults are DEER_SOLVE_OPTS_DEFAULT."""
    _fields_ = [("damping", ctypes.c_float), ("scan_f64", ctypes.c_int), ("multi_launch", ctypes.c_int),
                ("stall_window", ctypes.c_int), ("stall_escalate", ctypes.c_int)]


STALL_WINDOW_DEFAULT = 16


def solve_opts(damping: float = 0.0, scan_f64: bool = False, multi_launch: bool = False,
               stall_window: int = STALL_WINDOW_DEFAULT, stall_escalate: bool = True) -> SolveOpts:
    return SolveOpts(float(damping), int(bool(scan_f64)), int(bool(multi_launch)), int(stall_window),
                     int(bool(stall_escalate)))


class CellParams(ctypes.Structure):
    _fields_ = [("cell", ctypes.c_int), ("D", ctypes.c_int), ("M", ctypes.c_int),
                ("W", ctypes.c_void_p), ("U", ctypes.c_void_p), ("b", ctypes.c_void_p),
                ("b2", ctypes.c_void_p)]


_lib = None


def load_library():
    """Load libdeer.so (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  -- loads the HIP runtime torch uses first
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m evaluation_nonlinear_rnns_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    c_int, c_size, vp, fp = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
    sig = {
        "deer_workspace_size": ([ctypes.POINTER(CellParams), c_int, c_int, c_int, ctypes.POINTER(SolveOpts),
                                 ctypes.POINTER(c_size)], c_int),
        "deer_workspace_init": ([vp, c_size, vp], c_int),
        "deer_solve": ([ctypes.POINTER(CellParams), vp, vp, c_int, c_int, c_int, fp, c_int, ctypes.POINTER(SolveOpts),
                        vp, vp, vp, vp, vp, vp, vp, c_size, vp], c_int),
        "linear_scan_workspace_size": ([c_int, c_int, c_int, c_int, ctypes.POINTER(c_size)], c_int),
        "linear_scan_diag": ([vp, vp, vp, vp, c_int, c_int, c_int, vp, c_size, vp], c_int),
        "linear_scan_diag_noalloc": ([vp, vp, vp, vp, c_int, c_int, c_int, vp], c_int),
        "linear_scan_dense": ([vp, vp, vp, vp, c_int, c_int, c_int, vp, c_size, vp], c_int),
        "deer_rollout_workspace_size": ([ctypes.POINTER(CellParams), c_int, c_int, ctypes.POINTER(c_size)], c_int),
        "deer_rollout": ([ctypes.POINTER(CellParams), vp, vp, c_int, c_int, vp, vp, c_size, vp], c_int),
        "deer_lle_workspace_size": ([ctypes.POINTER(CellParams), c_int, c_int, ctypes.POINTER(c_size)], c_int),
        "deer_lle": ([ctypes.POINTER(CellParams), vp, vp, vp, vp, c_int, c_int, vp, vp, c_size, vp], c_int),
        "deer_broyden_workspace_size": ([ctypes.POINTER(CellParams), c_int, c_int, ctypes.POINTER(BroydenOpts),
                                         ctypes.POINTER(c_size)], c_int),
        "deer_solve_broyden": ([ctypes.POINTER(CellParams), vp, vp, c_int, c_int, ctypes.POINTER(BroydenOpts), fp,
                                c_int, vp, vp, vp, vp, vp, vp, c_size, vp], c_int),
        "linear_scan_dplr_workspace_size": ([c_int, c_int, c_int, c_int, c_int, ctypes.POINTER(c_size)], c_int),
        "linear_scan_dplr": ([fp, vp, vp, vp, vp, vp, c_int, c_int, c_int, c_int, c_int, vp, c_size, vp], c_int),
        "deer_profile_enable": ([c_int], c_int),
        "deer_profile_read": ([c_int, ctypes.POINTER(ctypes.c_longlong), ctypes.POINTER(ctypes.c_double)], c_int),
        "deer_bandwidth_probe": ([vp, c_size, vp, c_size, vp], c_int),
        "deer_last_error": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _lib = lib
    return lib


def _check(rc: int, allow_nc: bool = False) -> int:
    if rc == DEER_OK or (allow_nc and rc == DEER_NOT_CONVERGED):
        return rc
    raise DeerError(rc, load_library().deer_last_error().decode())


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t, name, dtype=None, shape=None):
    """Device pointer of a contiguous float32 CUDA tensor (or None)."""
    import torch
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != (dtype or torch.float32):
        raise TypeError(f"{name} must be {dtype or torch.float32}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


@dataclass
class Cell:
    """Cell parameters on the device (float32, contiguous).

    tanh: ``W [D,D]``, ``U [D,M]``, ``b [D]`` or None.
    GRU:  ``W`` = W_hh ``[3D,D]``, ``U`` = W_ih ``[3D,M]``, ``b`` = b_ih, ``b2`` = b_hh.
    """

    cell: str
    W: "object"
    U: "object"
    b: "object" = None
    b2: "object" = None

    @property
    def D(self) -> int:
        return int(self.W.shape[1])

    @property
    def M(self) -> int:
        return int(self.U.shape[1])

    def params(self) -> CellParams:
        rows = 3 * self.D if self.cell == "gru" else self.D
        _dev(self.W, "W", shape=(rows, self.D))
        _dev(self.U, "U", shape=(rows, self.M))
        _dev(self.b, "b", shape=(rows,))
        if self.cell == "gru":
            _dev(self.b2, "b2", shape=(rows,))
        return CellParams(CELLS[self.cell], self.D, self.M, _dev(self.W, "W"), _dev(self.U, "U"),
                          _dev(self.b, "b"), _dev(self.b2, "b2") if self.cell == "gru" else None)


# ------------------------------------------------------------- workspaces

def deer_workspace_size(cell: Cell, B: int, T: int, mode: str, scan_f64: bool = False,
                        stall_window: int = STALL_WINDOW_DEFAULT, stall_escalate: bool = True) -> int:
    lib = load_library()
    n = ctypes.c_size_t(0)
    p = cell.params()
    o = solve_opts(scan_f64=scan_f64, stall_window=stall_window, stall_escalate=stall_escalate)
    _check(lib.deer_workspace_size(ctypes.byref(p), B, T, MODES[mode], ctypes.byref(o), ctypes.byref(n)))
    return int(n.value)


def linear_scan_workspace_size(B: int, T: int, D: int, dense: bool = False) -> int:
    lib = load_library()
    n = ctypes.c_size_t(0)
    _check(lib.linear_scan_workspace_size(B, T, D, int(dense), ctypes.byref(n)))
    return int(n.value)


def new_workspace(nbytes: int, device=None):
    """A zero-filled, 256-byte aligned device workspace (torch allocation)."""
    import torch
    n = max(int(nbytes), 256)
    ws = torch.zeros(n, dtype=torch.uint8, device=device or "cuda")
    if ws.data_ptr() % 256 != 0:
        raise RuntimeError("workspace allocation is not 256-byte aligned")
    return ws


def deer_workspace_init(ws, stream=None) -> None:
    lib = load_library()
    _check(lib.deer_workspace_init(_dev(ws, "workspace", dtype=ws.dtype), ws.numel() * ws.element_size(),
                                   _stream(stream)))


# ---------------------------------------------------------------- solvers

def deer_solve(cell: Cell, x, s0=None, mode: str = "dense", tol: float = 1e-6, max_iter: int = 100,
               init_guess=None, out=None, workspace=None, stream=None, scan_f64: bool = False,
               damping: float = 0.0, multi_launch: bool = False, stall_window: int = STALL_WINDOW_DEFAULT,
               stall_escalate: bool = True, rms: bool = False):
    """Parallel fixed-point solve; returns ``(traj, iters, resid, status, rc)``,
    plus the per-sequence root-mean-square residual with ``rms=True``.

    ``mode``: ``"dense"`` (Newton), ``"diag"`` (diagonal quasi-Newton),
    ``"jacobi"`` or ``"picard"``; ``damping`` k shrinks the dense / diag blocks
    to ``(1 - k) J``.  ``traj`` is a ``[B,T,D]`` CUDA tensor; ``iters``,
    ``status`` are numpy int32 ``[B]``, ``resid`` numpy float32 ``[B]``; ``rc``
    is DEER_OK or DEER_NOT_CONVERGED.  ``scan_f64`` (dense mode) accumulates
    the linear solve in double precision from the start.  ``multi_launch``
    keeps small tanh problems (D <= 4, T <= 1024) on the multi-launch loop
    instead of the single-launch path.  ``stall_window`` / ``stall_escalate``:
    the finite-step check of ``deer_solve_opts_t`` (0 turns it off).
    """
    import numpy as np
    import torch
    lib = load_library()
    B, T, M = (int(v) for v in x.shape)
    D = cell.D
    if M != cell.M:
        raise ValueError(f"x has input size {M}, the cell expects {cell.M}")
    p = cell.params()
    o = solve_opts(damping, scan_f64, multi_launch, stall_window, stall_escalate)
    if out is None:
        out = torch.empty((B, T, D), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = new_workspace(deer_workspace_size(cell, B, T, mode, scan_f64, stall_window, stall_escalate),
                                  device=x.device)
    iters = np.zeros(B, np.int32)
    resid = np.zeros(B, np.float32)
    rms_a = np.zeros(B, np.float32)
    status = np.zeros(B, np.int32)
    rc = lib.deer_solve(ctypes.byref(p), _dev(x, "x", shape=(B, T, M)), _dev(s0, "s0", shape=(B, D)), B, T,
                        MODES[mode], ctypes.c_float(tol), int(max_iter), ctypes.byref(o),
                        _dev(init_guess, "init_guess", shape=(B, T, D)), _dev(out, "out", shape=(B, T, D)),
                        iters.ctypes.data_as(ctypes.c_void_p), resid.ctypes.data_as(ctypes.c_void_p),
                        rms_a.ctypes.data_as(ctypes.c_void_p) if rms else None,
                        status.ctypes.data_as(ctypes.c_void_p),
                        _dev(workspace, "workspace", dtype=workspace.dtype),
                        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, allow_nc=True)
    if rms:
        return out, iters, resid, status, rc, rms_a
    return out, iters, resid, status, rc


def linear_scan_diag(a, b, s0=None, out=None, workspace=None, stream=None):
    """``s_t = a_t * s_{t-1} + b_t`` over ``[B,T,D]`` tensors; returns ``s``."""
    import torch
    lib = load_library()
    B, T, D = (int(v) for v in a.shape)
    if out is None:
        out = torch.empty_like(a)
    if workspace is None:
        workspace = new_workspace(linear_scan_workspace_size(B, T, D), device=a.device)
    _check(lib.linear_scan_diag(_dev(a, "a"), _dev(b, "b", shape=(B, T, D)), _dev(s0, "s0", shape=(B, D)),
                                _dev(out, "out", shape=(B, T, D)), B, T, D,
                                _dev(workspace, "workspace", dtype=workspace.dtype),
                                workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


DEER_NOALLOC_SCRATCH_BYTES = 64 << 20


def linear_scan_diag_noalloc(a, b, s0=None, out=None, stream=None):
    """``linear_scan_diag`` without a workspace: the look-back state lives in the
    library's static device array (``DEER_NOALLOC_SCRATCH_BYTES``); ``out`` must be
    given by callers that cannot allocate.  Returns ``s``."""
    import torch
    lib = load_library()
    B, T, D = (int(v) for v in a.shape)
    if out is None:
        out = torch.empty_like(a)
    _check(lib.linear_scan_diag_noalloc(_dev(a, "a"), _dev(b, "b", shape=(B, T, D)), _dev(s0, "s0", shape=(B, D)),
                                        _dev(out, "out", shape=(B, T, D)), B, T, D, _stream(stream)))
    return out


def linear_scan_dense(A, b, s0=None, out=None, workspace=None, stream=None):
    """``s_t = A_t s_{t-1} + b_t`` with ``A [B,T,D,D]``; returns ``s [B,T,D]``."""
    import torch
    lib = load_library()
    B, T, D = (int(v) for v in b.shape)
    if out is None:
        out = torch.empty_like(b)
    if workspace is None:
        workspace = new_workspace(linear_scan_workspace_size(B, T, D, dense=True), device=b.device)
    _check(lib.linear_scan_dense(_dev(A, "A", shape=(B, T, D, D)), _dev(b, "b"), _dev(s0, "s0", shape=(B, D)),
                                 _dev(out, "out", shape=(B, T, D)), B, T, D,
                                 _dev(workspace, "workspace", dtype=workspace.dtype),
                                 workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def rollout_workspace_size(cell: Cell, B: int, T: int) -> int:
    lib = load_library()
    n = ctypes.c_size_t(0)
    p = cell.params()
    _check(lib.deer_rollout_workspace_size(ctypes.byref(p), B, T, ctypes.byref(n)))
    return int(n.value)


def deer_rollout(cell: Cell, x, s0=None, out=None, workspace=None, stream=None):
    """Sequential rollout on the GPU; returns ``traj [B,T,D]``."""
    import torch
    lib = load_library()
    B, T, M = (int(v) for v in x.shape)
    p = cell.params()
    if out is None:
        out = torch.empty((B, T, cell.D), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = new_workspace(rollout_workspace_size(cell, B, T), device=x.device)
    _check(lib.deer_rollout(ctypes.byref(p), _dev(x, "x", shape=(B, T, M)), _dev(s0, "s0", shape=(B, cell.D)),
                            B, T, _dev(out, "out", shape=(B, T, cell.D)),
                            _dev(workspace, "workspace", dtype=workspace.dtype),
                            workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def deer_lle(cell: Cell, x, traj, v0, s0=None, out=None, workspace=None, stream=None):
    """Largest Lyapunov exponent per sequence along ``traj [B,T,D]``; returns a
    float64 CUDA tensor ``[B]``.  ``v0 [B,D]`` are the probe vectors."""
    import torch
    lib = load_library()
    B, T, M = (int(v) for v in x.shape)
    D = cell.D
    p = cell.params()
    if out is None:
        out = torch.empty(B, dtype=torch.float64, device=x.device)
    if workspace is None:
        n = ctypes.c_size_t(0)
        _check(lib.deer_lle_workspace_size(ctypes.byref(p), B, T, ctypes.byref(n)))
        workspace = new_workspace(n.value, device=x.device)
    _check(lib.deer_lle(ctypes.byref(p), _dev(x, "x", shape=(B, T, M)), _dev(s0, "s0", shape=(B, D)),
                        _dev(traj, "traj", shape=(B, T, D)), _dev(v0, "v0", shape=(B, D)), B, T,
                        _dev(out, "out", dtype=torch.float64, shape=(B,)),
                        _dev(workspace, "workspace", dtype=workspace.dtype),
                        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def _broyden_opts(rank, multisecant, alpha, damping, gram_reg, chunk, sketch, D, stall_window):
    if rank > 0 and sketch is None:
        raise ValueError("a sketch [D, rank] is required for rank > 0")
    sk = _dev(sketch, "sketch", shape=(D, rank)) if rank > 0 else None
    return BroydenOpts(int(rank), int(bool(multisecant)), float(alpha), float(damping), float(gram_reg), int(chunk),
                       sk, int(stall_window))


def deer_broyden_workspace_size(cell: Cell, B: int, T: int, rank: int = 2, multisecant: bool = False,
                                chunk: int = 32) -> int:
    lib = load_library()
    n = ctypes.c_size_t(0)
    p = cell.params()
    o = BroydenOpts(int(rank), int(bool(multisecant)), 0.0, 0.0, 0.0, int(chunk), None, 0)
    _check(lib.deer_broyden_workspace_size(ctypes.byref(p), B, T, ctypes.byref(o), ctypes.byref(n)))
    return int(n.value)


def deer_solve_broyden(cell: Cell, x, sketch=None, s0=None, rank: int = 2, multisecant: bool = False,
                       alpha: float = 0.0, damping: float = 0.0, gram_reg: float = 0.0, chunk: int = 32,
                       tol: float = 1e-6, max_iter: int = 100, init_guess=None, out=None, workspace=None,
                       stream=None, stall_window: int = STALL_WINDOW_DEFAULT):
    """Parallel Broyden solve; returns ``(traj, iters, resid, status, rc)`` like
    :func:`deer_solve`.  ``sketch`` is a ``[D, rank]`` CUDA tensor."""
    import numpy as np
    import torch
    lib = load_library()
    B, T, M = (int(v) for v in x.shape)
    D = cell.D
    if M != cell.M:
        raise ValueError(f"x has input size {M}, the cell expects {cell.M}")
    p = cell.params()
    o = _broyden_opts(rank, multisecant, alpha, damping, gram_reg, chunk, sketch, D, stall_window)
    if out is None:
        out = torch.empty((B, T, D), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = new_workspace(deer_broyden_workspace_size(cell, B, T, rank, multisecant, chunk),
                                  device=x.device)
    iters = np.zeros(B, np.int32)
    resid = np.zeros(B, np.float32)
    status = np.zeros(B, np.int32)
    rc = lib.deer_solve_broyden(ctypes.byref(p), _dev(x, "x", shape=(B, T, M)), _dev(s0, "s0", shape=(B, D)), B, T,
                                ctypes.byref(o), ctypes.c_float(tol), int(max_iter),
                                _dev(init_guess, "init_guess", shape=(B, T, D)), _dev(out, "out", shape=(B, T, D)),
                                iters.ctypes.data_as(ctypes.c_void_p), resid.ctypes.data_as(ctypes.c_void_p),
                                status.ctypes.data_as(ctypes.c_void_p),
                                _dev(workspace, "workspace", dtype=workspace.dtype),
                                workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, allow_nc=True)
    return out, iters, resid, status, rc


def linear_scan_dplr_workspace_size(B: int, T: int, D: int, rank: int, chunk: int = 32) -> int:
    lib = load_library()
    n = ctypes.c_size_t(0)
    _check(lib.linear_scan_dplr_workspace_size(B, T, D, rank, chunk, ctypes.byref(n)))
    return int(n.value)


def linear_scan_dplr(alpha: float, U, V, c, sketch, chunk: int = 32, out=None, workspace=None, stream=None):
    """``delta_t = (alpha I + U_t V_t^T) delta_{t-1} + c_t`` with chunk carries
    re-compressed; ``U, V [B,T,rank,D]``, ``c [B,T,D]``, ``sketch [D, rank]``."""
    import torch
    lib = load_library()
    B, T, D = (int(v) for v in c.shape)
    rank = int(U.shape[2])
    if out is None:
        out = torch.empty_like(c)
    if workspace is None:
        workspace = new_workspace(linear_scan_dplr_workspace_size(B, T, D, rank, chunk), device=c.device)
    _check(lib.linear_scan_dplr(ctypes.c_float(alpha), _dev(U, "U", shape=(B, T, rank, D)),
                                _dev(V, "V", shape=(B, T, rank, D)), _dev(c, "c"),
                                _dev(sketch, "sketch", shape=(D, rank)), _dev(out, "out", shape=(B, T, D)),
                                B, T, D, rank, int(chunk), _dev(workspace, "workspace", dtype=workspace.dtype),
                                workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def deer_profile_enable(enable: bool = True) -> None:
    _check(load_library().deer_profile_enable(int(enable)))


def deer_profile_read(which: int) -> Tuple[int, float]:
    """``(launches, milliseconds)`` timed for a kernel class since the last read."""
    n = ctypes.c_longlong(0)
    ms = ctypes.c_double(0.0)
    _check(load_library().deer_profile_read(int(which), ctypes.byref(n), ctypes.byref(ms)))
    return int(n.value), float(ms.value)


PROFILE_EVAL, PROFILE_SCAN, PROFILE_PROJECTION, PROFILE_CHECK, PROFILE_COMPOSE = 0, 1, 2, 3, 4


def bandwidth_probe(src, dst, stream=None) -> None:
    """Stream all of ``src`` into ``dst`` (contiguous CUDA tensors; ``src``
    1, 2, 4 or 8 times the bytes of ``dst``) with the library's probe kernel:
    output vector i is the XOR of the input vectors i, i + n, ... (a bandwidth
    reference; a copy when the sizes are equal)."""
    import torch
    st = stream if stream is not None else torch.cuda.current_stream()
    _check(load_library().deer_bandwidth_probe(ctypes.c_void_p(src.data_ptr()), src.numel() * src.element_size(),
                                               ctypes.c_void_p(dst.data_ptr()), dst.numel() * dst.element_size(),
                                               ctypes.c_void_p(st.cuda_stream)))


def cell_from_problem(p: dict, device="cuda") -> Cell:
    """Move a problem's float32 parameters (``inputs`` module) to the device."""
    import torch

    def t(a):
        return None if a is None else torch.from_numpy(a).to(device)

    return Cell(p["cell"], t(p["W"]), t(p["U"]), t(p.get("b")), t(p.get("b2")) if p["cell"] == "gru" else None)
