"""Python binding of libdion: one Dion / Orth-Dion optimizer step on an
MI355X (gfx950), through the C ABI of include/dion.h.

This module only marshals arguments (ctypes): torch tensors supply device
memory and the current HIP stream, and every part of the step runs in
libdion's HIP kernels.  There is no CPU or PyTorch fallback: calls raise
when the built library is missing.

    import rank_orthonormalized_optimizer_dion_amd as dion
    ws = dion.step(X, G, R, V, eta=0.01, beta=0.95, variant="orth")
    dion.check_status(ws, 1)        # optional: waits, raises on breakdown
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

__all__ = [
    "DionError", "Breakdown", "Plan", "load", "library_path", "workspace_size",
    "workspace_size_batched", "step", "step_batched", "step_noalloc", "status",
    "check_status", "version", "VARIANTS",
]

OK = 0
ERR_INVALID_ARG = -1
ERR_WORKSPACE = -2
ERR_HIP = -3
ERR_BREAKDOWN = -4

VARIANTS = {"dion": 0, "orth": 1}
MATH = {"f32": 0x000, "bf16x3": 0x100}
SHARDED = 0x200
GRAM_F64 = 0x400   # OR into math: float64 MFMA Gram matrix instead of sliced int8
SCHED_GROUPED = 0x800   # OR into math: small matrices through the grouped schedule too
SHARD_GRAM, SHARD_W = 0, 1
BUF_W, BUF_P, BUF_U = 1, 2, 3   # dion_plan_buffer: intermediate factors of the last step
STATUS_ORTH_P, STATUS_ORTH_W, STATUS_COLNORM = 1, 2, 4

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB: Optional[ctypes.CDLL] = None


def library_path() -> str:
    return os.environ.get("LIBDION_PATH", os.path.join(_HERE, "libdion.so"))


class DionError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libdion error {code}: {msg}")
        self.code = code


class Breakdown(DionError):
    """The step hit a numerical breakdown; X, R, V were left unchanged."""

    def __init__(self, code: int, msg: str, per_matrix: List[int]):
        super().__init__(code, msg)
        self.per_matrix = per_matrix


class dion_matrix(ctypes.Structure):
    _fields_ = [("X", ctypes.c_void_p), ("G", ctypes.c_void_p), ("R", ctypes.c_void_p),
                ("V", ctypes.c_void_p), ("m", ctypes.c_int64), ("n", ctypes.c_int64),
                ("r", ctypes.c_int64)]


def load() -> ctypes.CDLL:
    """Load libdion.so (built by ``build.py``); raises if it is missing."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"libdion is not built ({path} missing); run "
            "`python -m rank_orthonormalized_optimizer_dion_amd.build`")
    lib = ctypes.CDLL(path)
    c_size, c_int, c_i64, c_f, vp = (ctypes.c_size_t, ctypes.c_int, ctypes.c_int64,
                                     ctypes.c_float, ctypes.c_void_p)
    mats_p = ctypes.POINTER(dion_matrix)
    sig = {
        "dion_version": (c_int, []),
        "dion_error_string": (ctypes.c_char_p, [c_int]),
        "dion_workspace_size": (c_size, [c_i64, c_i64, c_i64, c_int, c_int]),
        "dion_step": (c_int, [vp, vp, vp, vp, c_i64, c_i64, c_i64, c_f, c_f, c_int, c_int,
                              vp, c_size, vp]),
        "dion_workspace_size_batched": (c_size, [mats_p, c_int, c_int, c_int]),
        "dion_step_batched": (c_int, [mats_p, c_int, c_f, c_f, c_int, c_int, vp, c_size, vp]),
        "dion_plan_create": (c_int, [mats_p, c_int, c_int, c_int, ctypes.POINTER(vp)]),
        "dion_plan_workspace_size": (c_size, [vp]),
        "dion_plan_count": (c_int, [vp]),
        "dion_plan_step": (c_int, [vp, c_f, c_f, vp, c_size, vp]),
        "dion_plan_destroy": (None, [vp]),
        "dion_status": (c_int, [vp, c_int, vp, ctypes.POINTER(c_int)]),
        "dion_plan_timing_enable": (c_int, [vp, c_int]),
        "dion_plan_timing_read": (c_int, [vp, ctypes.POINTER(ctypes.c_double),
                                          ctypes.POINTER(c_int)]),
        "dion_plan_shard_stage": (c_int, [vp, c_int, c_f, c_f, vp, c_size, vp]),
        "dion_plan_shard_buffer": (c_int, [vp, c_int, c_int, ctypes.POINTER(c_size),
                                           ctypes.POINTER(c_size)]),
        "dion_plan_buffer": (c_int, [vp, c_int, c_int, ctypes.POINTER(c_size),
                                     ctypes.POINTER(c_size)]),
        "dion_step_noalloc": (c_int, [vp, vp, vp, vp, c_i64, c_i64, c_i64, c_f, c_f, c_int,
                                      c_int, vp, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def version() -> int:
    return load().dion_version()


def _err(code: int) -> DionError:
    msg = load().dion_error_string(code).decode()
    return DionError(code, msg)


def _variant(v, math="f32") -> int:
    """Rule (``"dion"`` / ``"orth"`` or its code) OR-ed with the math mode
    (``"f32"``: float32 MFMA products; ``"bf16x3"``: split-bfloat16)."""
    if isinstance(v, str):
        if v not in VARIANTS:
            raise ValueError(f"variant must be one of {list(VARIANTS)}")
        v = VARIANTS[v]
    if isinstance(math, str):
        if math not in MATH:
            raise ValueError(f"math must be one of {list(MATH)}")
        math = MATH[math]
    return int(v) | int(math)


def _torch():
    import torch
    return torch


def _gdtype(G) -> int:
    torch = _torch()
    if G.dtype == torch.float32:
        return 0
    if G.dtype == torch.bfloat16:
        return 1
    raise TypeError("G must be float32 or bfloat16")


def _stream_handle(stream, device) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream)


def _check(X, G, R, V):
    torch = _torch()
    for name, t in (("X", X), ("G", G), ("R", R), ("V", V)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous (row-major)")
        if t.dim() != 2:
            raise ValueError(f"{name} must be 2-D")
    for name, t in (("X", X), ("R", R), ("V", V)):
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    m, n = X.shape
    if tuple(G.shape) != (m, n) or tuple(R.shape) != (m, n) or V.shape[0] != n:
        raise ValueError("shape mismatch: X, G, R are m x n and V is n x r")
    return m, n, V.shape[1]


def workspace_size(m: int, n: int, r: int, variant="orth", g_dtype=None, math="f32") -> int:
    torch = _torch()
    gd = 1 if g_dtype == torch.bfloat16 else 0
    size = load().dion_workspace_size(m, n, r, _variant(variant, math), gd)
    if size == 0:
        raise ValueError("invalid shape or rank")
    return int(size)


def _workspace(nbytes: int, device, workspace):
    torch = _torch()
    if workspace is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace too small: need {nbytes} bytes")
    return workspace


def step(X, G, R, V, eta: float, beta: float, variant="orth", workspace=None, stream=None,
         math="f32"):
    """One step on one matrix, enqueued on `stream` (default: current).

    X, R, V (float32) are updated in place; G (float32 or bfloat16) is read.
    Returns the workspace tensor (pass it back to reuse it, or to
    ``status``)."""
    m, n, r = _check(X, G, R, V)
    lib = load()
    gd, var = _gdtype(G), _variant(variant, math)
    nbytes = lib.dion_workspace_size(m, n, r, var, gd)
    if nbytes == 0:
        raise _err(ERR_INVALID_ARG)
    ws = _workspace(nbytes, X.device, workspace)
    rc = lib.dion_step(X.data_ptr(), G.data_ptr(), R.data_ptr(), V.data_ptr(), m, n, r,
                       float(eta), float(beta), var, gd, ws.data_ptr(), nbytes,
                       _stream_handle(stream, X.device))
    if rc != OK:
        raise _err(rc)
    return ws


def step_noalloc(X, G, R, V, eta: float, beta: float, variant="orth", status_out=None,
                 stream=None, math="f32"):
    """One step on one matrix with the library's own scratch (no workspace
    argument; dion_step_noalloc).  status_out: optional int32 GPU tensor of
    one element that receives the matrix's status word."""
    m, n, r = _check(X, G, R, V)
    lib = load()
    if status_out is not None and (not status_out.is_cuda or status_out.numel() < 1 or
                                   status_out.dtype != _torch().int32):
        raise ValueError("status_out must be an int32 GPU tensor")
    rc = lib.dion_step_noalloc(X.data_ptr(), G.data_ptr(), R.data_ptr(), V.data_ptr(), m, n, r,
                               float(eta), float(beta), _variant(variant, math), _gdtype(G),
                               status_out.data_ptr() if status_out is not None else None,
                               _stream_handle(stream, X.device))
    if rc != OK:
        raise _err(rc)


def _mat_array(mats: Sequence[Tuple]) -> Tuple[ctypes.Array, int]:
    if len(mats) == 0:
        raise ValueError("empty matrix list")
    gd = None
    arr = (dion_matrix * len(mats))()
    for i, (X, G, R, V) in enumerate(mats):
        m, n, r = _check(X, G, R, V)
        g = _gdtype(G)
        if gd is None:
            gd = g
        elif g != gd:
            raise TypeError("every G of a grouped step must have the same dtype")
        arr[i] = dion_matrix(X.data_ptr(), G.data_ptr(), R.data_ptr(), V.data_ptr(), m, n, r)
    return arr, gd


def workspace_size_batched(mats: Sequence[Tuple], variant="orth", math="f32") -> int:
    arr, gd = _mat_array(mats)
    size = load().dion_workspace_size_batched(arr, len(mats), _variant(variant, math), gd)
    if size == 0:
        raise _err(ERR_INVALID_ARG)
    return int(size)


def step_batched(mats: Sequence[Tuple], eta: float, beta: float, variant="orth",
                 workspace=None, stream=None, math="f32"):
    """Grouped step over a list of (X, G, R, V) tuples; returns the workspace."""
    arr, gd = _mat_array(mats)
    lib = load()
    var = _variant(variant, math)
    nbytes = lib.dion_workspace_size_batched(arr, len(mats), var, gd)
    if nbytes == 0:
        raise _err(ERR_INVALID_ARG)
    dev = mats[0][0].device
    ws = _workspace(nbytes, dev, workspace)
    rc = lib.dion_step_batched(arr, len(mats), float(eta), float(beta), var, gd,
                               ws.data_ptr(), nbytes, _stream_handle(stream, dev))
    if rc != OK:
        raise _err(rc)
    return ws


class Plan:
    """A grouped step over a fixed list of matrices (dion_plan_*)."""

    def __init__(self, mats: Sequence[Tuple], variant="orth", math="f32", sharded=False):
        """sharded: the matrices are row shards of global matrices, stepped
        with dion_plan_shard_stage / shard_buffer (see include/dion.h)."""
        arr, gd = _mat_array(mats)
        self._lib = load()
        self._mats = list(mats)          # keep the tensors alive
        self.count = len(mats)
        self.device = mats[0][0].device
        h = ctypes.c_void_p()
        var = _variant(variant, math) | (SHARDED if sharded else 0)
        rc = self._lib.dion_plan_create(arr, self.count, var, gd, ctypes.byref(h))
        if rc != OK:
            raise _err(rc)
        self._h = h
        self.workspace_bytes = int(self._lib.dion_plan_workspace_size(h))

    def new_workspace(self):
        return _workspace(self.workspace_bytes, self.device, None)

    def step(self, eta: float, beta: float, workspace, stream=None):
        if self._h is None:
            raise RuntimeError("plan is closed")
        if workspace.numel() * workspace.element_size() < self.workspace_bytes:
            raise ValueError("workspace too small")
        rc = self._lib.dion_plan_step(self._h, float(eta), float(beta), workspace.data_ptr(),
                                      self.workspace_bytes, _stream_handle(stream, self.device))
        if rc != OK:
            raise _err(rc)

    def shard_stage(self, stage: int, eta: float, beta: float, workspace, stream=None):
        """Stage 0, 1 or 2 of a sharded step (dion_plan_shard_stage)."""
        if self._h is None:
            raise RuntimeError("plan is closed")
        if workspace.numel() * workspace.element_size() < self.workspace_bytes:
            raise ValueError("workspace too small")
        rc = self._lib.dion_plan_shard_stage(self._h, int(stage), float(eta), float(beta),
                                             workspace.data_ptr(), self.workspace_bytes,
                                             _stream_handle(stream, self.device))
        if rc != OK:
            raise _err(rc)

    def shard_buffer(self, workspace, which: int, index: int):
        """The exchange buffer `which` (SHARD_GRAM: float64 rp x rp; SHARD_W:
        float32 n x r) of matrix `index`, as a view into `workspace`."""
        torch = _torch()
        off, nbytes = ctypes.c_size_t(), ctypes.c_size_t()
        rc = self._lib.dion_plan_shard_buffer(self._h, int(which), int(index), ctypes.byref(off),
                                              ctypes.byref(nbytes))
        if rc != OK:
            raise _err(rc)
        raw = workspace.view(torch.uint8)[off.value:off.value + nbytes.value]
        if which == SHARD_GRAM:
            rp = int(round((nbytes.value // 8) ** 0.5))
            return raw.view(torch.float64).view(rp, rp)
        n, r = self._mats[index][3].shape
        return raw.view(torch.float32).view(n, r)

    def buffer(self, workspace, which: int, index: int):
        """Intermediate factor `which` (BUF_P: P = M V, BUF_U: U = orth(P),
        both m x r; BUF_W: W = M^T U, n x r; float32) of matrix `index` after
        the last step on `workspace`, as a view into it
        (dion_plan_buffer)."""
        torch = _torch()
        off, nbytes = ctypes.c_size_t(), ctypes.c_size_t()
        rc = self._lib.dion_plan_buffer(self._h, int(which), int(index), ctypes.byref(off),
                                        ctypes.byref(nbytes))
        if rc != OK:
            raise _err(rc)
        raw = workspace.view(torch.uint8)[off.value:off.value + nbytes.value]
        X, V = self._mats[index][0], self._mats[index][3]
        rows = V.shape[0] if which == BUF_W else X.shape[0]
        return raw.view(torch.float32).view(rows, V.shape[1])

    PHASES = ("mv", "orth_p", "mtu", "right", "update")

    def timing_enable(self, max_steps: int) -> None:
        """Record per-phase HIP events on the next `max_steps` steps."""
        rc = self._lib.dion_plan_timing_enable(self._h, int(max_steps))
        if rc != OK:
            raise _err(rc)

    def timing_read(self):
        """Wait for the recorded steps; return ({phase: summed ms}, steps)."""
        ms = (ctypes.c_double * len(self.PHASES))()
        steps = ctypes.c_int()
        rc = self._lib.dion_plan_timing_read(self._h, ms, ctypes.byref(steps))
        if rc != OK:
            raise _err(rc)
        return dict(zip(self.PHASES, list(ms))), steps.value

    def close(self):
        if getattr(self, "_h", None) is not None:
            self._lib.dion_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def status(workspace, count: int, stream=None) -> Tuple[int, List[int]]:
    """Wait for `stream`; return (code, per-matrix DION_STATUS_* flags)."""
    lib = load()
    per = (ctypes.c_int * count)()
    rc = lib.dion_status(workspace.data_ptr(), count,
                         _stream_handle(stream, workspace.device), per)
    if rc not in (OK, ERR_BREAKDOWN):
        raise _err(rc)
    return rc, list(per)


def check_status(workspace, count: int, stream=None) -> None:
    """Raise Breakdown if the last step on `workspace` broke down."""
    rc, per = status(workspace, count, stream)
    if rc == ERR_BREAKDOWN:
        raise Breakdown(rc, load().dion_error_string(rc).decode(), per)

