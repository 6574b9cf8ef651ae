"""Thin Python binding of libpararnn.so (argument marshalling only).

Every step of the solve runs in the HIP library; this module only checks
tensor placement, allocates outputs and workspace with torch, and passes raw
device pointers plus torch's current HIP stream through ctypes. There is no
fallback: if the library is missing or the tensors are not on a ROCm device,
the call raises.
"""
from __future__ import annotations

import ctypes
import re
from pathlib import Path
from typing import Optional, Sequence

import torch

PKG = Path(__file__).resolve().parent
LIB_PATH = PKG / "libpararnn.so"
HEADER = PKG.parent / "include" / "pararnn.h"

GRU, LSTM = 0, 1
OP_SOLVE, OP_ADJOINT, OP_SCAN_DIAG, OP_SCAN_BLOCK2, OP_SCAN_DENSE = 0, 1, 2, 3, 4
F32, BF16 = 0, 1
CELLS = {"gru": GRU, "lstm": LSTM}
GATES = {"gru": 3, "lstm": 4}
NSTATE = {"gru": 1, "lstm": 2}


class PararnnError(RuntimeError):
    pass


class Opts(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32),
        ("L", ctypes.c_int32),
        ("D", ctypes.c_int32),
        ("max_iters", ctypes.c_int32),
        ("tol", ctypes.c_float),
        ("early_exit", ctypes.c_int32),
        ("u_dtype", ctypes.c_int32),
        ("events", ctypes.c_void_p),
        ("schedule", ctypes.c_int32),
    ]


SCHEDULES = {"auto": 0, "fused": 1, "per_iteration": 2}


class Plan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("vec", "chunk", "channels", "nchunks", "tiles_per_row", "inclusive_only", "fused")]


def header_functions() -> list[str]:
    """Names of the functions declared in include/pararnn.h."""
    text = HEADER.read_text()
    return re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?(pararnn_[a-z_0-9]+)\s*\(", text, re.M)


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise PararnnError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(str(LIB_PATH))
        P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        OPTP = ctypes.POINTER(Opts)
        L.pararnn_workspace_bytes.argtypes = [I32, I32, OPTP]
        L.pararnn_workspace_bytes.restype = SZ
        L.pararnn_solve_gru.argtypes = [P, P, P, P, P, SZ, OPTP, P, P, P, P]
        L.pararnn_solve_gru.restype = I32
        L.pararnn_solve_gru_scratch.argtypes = [P, P, P, P, OPTP, P, P, P, P]
        L.pararnn_solve_gru_scratch.restype = I32
        L.pararnn_scratch_bytes.argtypes = []
        L.pararnn_scratch_bytes.restype = SZ
        L.pararnn_solve_lstm.argtypes = [P, P, P, P, P, P, P, SZ, OPTP, P, P, P, P]
        L.pararnn_solve_lstm.restype = I32
        L.pararnn_adjoint.argtypes = [I32, P, P, P, P, P, P, P, P, P, P, P, SZ, OPTP, P]
        L.pararnn_adjoint.restype = I32
        L.pararnn_scan_diag.argtypes = [P, P, P, P, P, SZ, OPTP, P]
        L.pararnn_scan_diag.restype = I32
        L.pararnn_scan_block2.argtypes = [P, P, P, P, P, SZ, OPTP, P]
        L.pararnn_scan_block2.restype = I32
        L.pararnn_scan_dense.argtypes = [P, P, P, P, P, SZ, OPTP, P]
        L.pararnn_scan_dense.restype = I32
        L.pararnn_plan_query.argtypes = [I32, I32, OPTP, ctypes.POINTER(Plan)]
        L.pararnn_plan_query.restype = I32
        L.pararnn_strerror.argtypes = [I32]
        L.pararnn_strerror.restype = ctypes.c_char_p
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().pararnn_strerror(status).decode()


def _check(status: int, what: str):
    if status != 0:
        raise PararnnError(f"{what} failed: {status} ({strerror(status)})")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise PararnnError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise PararnnError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise PararnnError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise PararnnError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _u_dtype(u: torch.Tensor) -> int:
    if u.dtype == torch.float32:
        return F32
    if u.dtype == torch.bfloat16:
        return BF16
    raise PararnnError(f"u must be float32 or bfloat16, got {u.dtype}")


def make_opts(B, L, D, iters=3, tol=1e-4, early_exit=False, u_dtype=BF16, events=None, schedule="auto"):
    o = Opts(B, L, D, iters, tol, int(bool(early_exit)), u_dtype, None, SCHEDULES[schedule])
    keep = None
    if events is not None:
        keep = (ctypes.c_void_p * len(events))(*events)
        o.events = ctypes.cast(keep, ctypes.c_void_p)
    return o, keep


def workspace_bytes(cell: str, op: int, B: int, L: int, D: int, iters: int = 3,
                    u_dtype: int = BF16) -> int:
    o, _ = make_opts(B, L, D, iters, 1e-4, False, u_dtype)
    return int(lib().pararnn_workspace_bytes(CELLS[cell], op, ctypes.byref(o)))


def plan(cell: str, op: int, B: int, L: int, D: int, iters: int = 3, u_dtype: int = BF16,
         schedule: str = "auto", early_exit: bool = False) -> dict:
    """The launch plan of a call (pararnn_plan_query; host-only): chunk length,
    channels per workgroup, chunk count, workgroups per chunk row, and whether
    the chunk carry runs in the inclusive-only (bitwise-reproducible) mode."""
    o, _ = make_opts(B, L, D, iters, 1e-4, early_exit, u_dtype, None, schedule)
    pl = Plan()
    _check(lib().pararnn_plan_query(CELLS.get(cell, GRU), op, ctypes.byref(o), ctypes.byref(pl)),
           "pararnn_plan_query")
    return {n: int(getattr(pl, n)) for n, _ in Plan._fields_}


def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    # torch's caching allocator returns 512-byte aligned blocks
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def solve(cell: str, u: torch.Tensor, a: torch.Tensor, *, h0=None, c0=None, iters: int = 3,
          tol: float = 1e-4, early_exit: bool = False, ws: Optional[torch.Tensor] = None,
          out=None, events: Optional[Sequence[int]] = None, schedule: str = "auto"):
    """Newton solve; returns dict(h, c (LSTM), iters, converged, max_update) on u's device."""
    G, NS = GATES[cell], NSTATE[cell]
    _dev(u, "u")
    if u.dim() != 4 or u.shape[2] != G:
        raise PararnnError(f"u must be [B][L][{G}][D]")
    B, L, _, D = u.shape
    dev = u.device
    _dev(a, "a", torch.float32, (G, D))
    _dev(h0, "h0", torch.float32, (B, D))
    _dev(c0, "c0", torch.float32, (B, D))
    udt = _u_dtype(u)
    if out is None:
        out = {"h": torch.empty(B, L, D, dtype=torch.float32, device=dev)}
        if NS == 2:
            out["c"] = torch.empty(B, L, D, dtype=torch.float32, device=dev)
    for k in out:
        _dev(out[k], k, torch.float32, (B, L, D))
    it = torch.empty(1, dtype=torch.int32, device=dev)
    conv = torch.empty(B, dtype=torch.int32, device=dev)
    mu = torch.empty(iters, B, dtype=torch.float32, device=dev)
    o, keep = make_opts(B, L, D, iters, tol, early_exit, udt, events, schedule)
    need = int(lib().pararnn_workspace_bytes(CELLS[cell], OP_SOLVE, ctypes.byref(o)))
    if need == 0:
        raise PararnnError("invalid sizes or iteration count")
    if ws is None:
        ws = alloc_workspace(need, dev)
    if cell == "gru":
        st = lib().pararnn_solve_gru(_ptr(u), _ptr(a), _ptr(h0), _ptr(out["h"]), _ptr(ws), ws.numel(),
                                     ctypes.byref(o), _ptr(it), _ptr(conv), _ptr(mu), _stream(dev))
    else:
        st = lib().pararnn_solve_lstm(_ptr(u), _ptr(a), _ptr(c0), _ptr(h0), _ptr(out["c"]), _ptr(out["h"]),
                                      _ptr(ws), ws.numel(), ctypes.byref(o), _ptr(it), _ptr(conv),
                                      _ptr(mu), _stream(dev))
    del keep
    _check(st, f"pararnn_solve_{cell}")
    res = dict(out)
    res.update(iters=it, converged=conv, max_update=mu, ws=ws)
    return res


def scratch_bytes() -> int:
    """Size of the scratch array built into the library (pararnn_solve_gru_scratch)."""
    return int(lib().pararnn_scratch_bytes())


def solve_gru_scratch(u: torch.Tensor, a: torch.Tensor, *, h0=None, iters: int = 3, tol: float = 1e-4,
                      early_exit: bool = False, out: Optional[torch.Tensor] = None, it=None, conv=None,
                      mu=None, events: Optional[Sequence[int]] = None, schedule: str = "auto"):
    """ParaGRU solve through pararnn_solve_gru_scratch: the library's built-in
    scratch replaces the workspace, so the call itself allocates nothing on the
    device when out, it, conv and mu are passed in. Returns dict(h, iters,
    converged, max_update)."""
    _dev(u, "u")
    if u.dim() != 4 or u.shape[2] != 3:
        raise PararnnError("u must be [B][L][3][D]")
    B, L, _, D = u.shape
    dev = u.device
    _dev(a, "a", torch.float32, (3, D))
    _dev(h0, "h0", torch.float32, (B, D))
    if out is None:
        out = torch.empty(B, L, D, dtype=torch.float32, device=dev)
    _dev(out, "h", torch.float32, (B, L, D))
    it = torch.empty(1, dtype=torch.int32, device=dev) if it is None else _dev(it, "iters", torch.int32, (1,))
    conv = (torch.empty(B, dtype=torch.int32, device=dev) if conv is None
            else _dev(conv, "converged", torch.int32, (B,)))
    mu = (torch.empty(iters, B, dtype=torch.float32, device=dev) if mu is None
          else _dev(mu, "max_update", torch.float32, (iters, B)))
    o, keep = make_opts(B, L, D, iters, tol, early_exit, _u_dtype(u), events, schedule)
    st = lib().pararnn_solve_gru_scratch(_ptr(u), _ptr(a), _ptr(h0), _ptr(out), ctypes.byref(o), _ptr(it),
                                         _ptr(conv), _ptr(mu), _stream(dev))
    del keep
    _check(st, "pararnn_solve_gru_scratch")
    return dict(h=out, iters=it, converged=conv, max_update=mu)


def solve_gru(u, a, h0=None, **kw):
    return solve("gru", u, a, h0=h0, **kw)


def solve_lstm(u, a, c0=None, h0=None, **kw):
    return solve("lstm", u, a, h0=h0, c0=c0, **kw)


def adjoint(cell: str, u: torch.Tensor, a: torch.Tensor, h: torch.Tensor, dh: torch.Tensor, *,
            c=None, h0=None, c0=None, want_ds0: bool = False, want_da: bool = False,
            ws: Optional[torch.Tensor] = None, du: Optional[torch.Tensor] = None,
            events: Optional[Sequence[int]] = None):
    """Reverse scan along the trajectory (c, h); returns dict(du, ds0, da)."""
    G, NS = GATES[cell], NSTATE[cell]
    _dev(u, "u")
    if u.dim() != 4 or u.shape[2] != G:
        raise PararnnError(f"u must be [B][L][{G}][D]")
    B, L, _, D = u.shape
    dev = u.device
    _dev(a, "a", torch.float32, (G, D))
    _dev(h, "h", torch.float32, (B, L, D))
    _dev(c, "c", torch.float32, (B, L, D))
    _dev(dh, "dh", torch.float32, (B, L, D))
    _dev(h0, "h0", torch.float32, (B, D))
    _dev(c0, "c0", torch.float32, (B, D))
    if NS == 2 and c is None:
        raise PararnnError("the LSTM adjoint needs the c trajectory")
    if du is None:
        du = torch.empty(B, L, G, D, dtype=torch.float32, device=dev)
    _dev(du, "du", torch.float32, (B, L, G, D))
    ds0 = torch.empty(NS, B, D, dtype=torch.float32, device=dev) if want_ds0 else None
    da = torch.empty(G, D, dtype=torch.float32, device=dev) if want_da else None
    o, keep = make_opts(B, L, D, 1, 0.0, False, _u_dtype(u), events)
    need = int(lib().pararnn_workspace_bytes(CELLS[cell], OP_ADJOINT, ctypes.byref(o)))
    if need == 0:
        raise PararnnError("invalid sizes")
    if ws is None:
        ws = alloc_workspace(need, dev)
    st = lib().pararnn_adjoint(CELLS[cell], _ptr(u), _ptr(a), _ptr(c0), _ptr(h0), _ptr(c), _ptr(h), _ptr(dh),
                               _ptr(du), _ptr(ds0), _ptr(da), _ptr(ws), ws.numel(), ctypes.byref(o),
                               _stream(dev))
    del keep
    _check(st, "pararnn_adjoint")
    return dict(du=du, ds0=ds0, da=da, ws=ws)


def scan(A: torch.Tensor, b: torch.Tensor, s0: Optional[torch.Tensor] = None, *,
         out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
         events: Optional[Sequence[int]] = None):
    """Linear recurrence s_l = A_l s_{l-1} + b_l per channel (pararnn_scan_diag
    or pararnn_scan_block2, chosen by the shape of A).

    Diagonal: A, b [B][L][D], s0 [B][D]. 2x2 blocks: A [2][2][B][L][D] (block
    rows first), b [2][B][L][D], s0 [2][B][D]. All fp32 device tensors; s0 may
    be None (zero). Returns dict(s, ws) with s shaped like b.
    """
    _dev(A, "A", torch.float32)
    if A.dim() == 3:
        ns, (B, L, D) = 1, A.shape
    elif A.dim() == 5 and tuple(A.shape[:2]) == (2, 2):
        ns, (B, L, D) = 2, A.shape[2:]
    else:
        raise PararnnError("A must be [B][L][D] or [2][2][B][L][D]")
    bshape = (B, L, D) if ns == 1 else (2, B, L, D)
    _dev(b, "b", torch.float32, bshape)
    _dev(s0, "s0", torch.float32, (B, D) if ns == 1 else (2, B, D))
    if out is None:
        out = torch.empty(bshape, dtype=torch.float32, device=A.device)
    _dev(out, "out", torch.float32, bshape)
    op = OP_SCAN_DIAG if ns == 1 else OP_SCAN_BLOCK2
    o, keep = make_opts(B, L, D, 1, 0.0, False, F32, events)
    need = int(lib().pararnn_workspace_bytes(GRU, op, ctypes.byref(o)))
    if need == 0:
        raise PararnnError("invalid sizes")
    if ws is None:
        ws = alloc_workspace(need, A.device)
    fn = lib().pararnn_scan_diag if ns == 1 else lib().pararnn_scan_block2
    st = fn(_ptr(A), _ptr(b), _ptr(s0), _ptr(out), _ptr(ws), ws.numel(), ctypes.byref(o), _stream(A.device))
    del keep
    _check(st, "pararnn_scan_diag" if ns == 1 else "pararnn_scan_block2")
    return dict(s=out, ws=ws)


def scan_dense(A: torch.Tensor, b: torch.Tensor, s0: Optional[torch.Tensor] = None, *,
               out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
               events: Optional[Sequence[int]] = None):
    """Linear recurrence with a dense n x n matrix per step (pararnn_scan_dense):
    A [B][L][n][n] (A_l[r][q] multiplies s_{l-1}[q] into s_l[r]), b [B][L][n],
    s0 [B][n] or None; fp32 device tensors, n <= 32. Returns dict(s, ws)."""
    _dev(A, "A", torch.float32)
    if A.dim() != 4 or A.shape[2] != A.shape[3]:
        raise PararnnError("A must be [B][L][n][n]")
    B, L, n = A.shape[:3]
    _dev(b, "b", torch.float32, (B, L, n))
    _dev(s0, "s0", torch.float32, (B, n))
    if out is None:
        out = torch.empty(B, L, n, dtype=torch.float32, device=A.device)
    _dev(out, "out", torch.float32, (B, L, n))
    o, keep = make_opts(B, L, n, 1, 0.0, False, F32, events)
    need = int(lib().pararnn_workspace_bytes(GRU, OP_SCAN_DENSE, ctypes.byref(o)))
    if need == 0:
        raise PararnnError("invalid sizes (the dense scan takes 1 <= n <= 32)")
    if ws is None:
        ws = alloc_workspace(need, A.device)
    st = lib().pararnn_scan_dense(_ptr(A), _ptr(b), _ptr(s0), _ptr(out), _ptr(ws), ws.numel(), ctypes.byref(o),
                                  _stream(A.device))
    del keep
    _check(st, "pararnn_scan_dense")
    return dict(s=out, ws=ws)
