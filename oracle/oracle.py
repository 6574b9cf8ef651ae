"""ctypes wrapper of the fp64 CPU oracle (pararnn_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only users. Nothing here touches the GPU or the HIP
library; inputs are numpy arrays (or anything numpy can convert), outputs are
float64 numpy arrays. See pararnn_oracle.c for the definitions and sources.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

HERE = Path(__file__).resolve().parent
SRC = HERE / "pararnn_oracle.c"
LIB = HERE / "liboracle.so"

CELLS = {"gru": 0, "lstm": 1}
GATES = {"gru": 3, "lstm": 4}
NSTATE = {"gru": 1, "lstm": 2}

_lib = None


def build(force: bool = True) -> Path:
    """Compile the oracle with gcc (plain -O2, no fast-math)."""
    if force or not LIB.exists():
        tmp = LIB.with_suffix(".so.tmp")
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
                        "-o", str(tmp), str(SRC), "-lm", "-lpthread"], check=True)
        os.replace(tmp, LIB)
    return LIB


def _bind(path):
    lib = ctypes.CDLL(str(path))
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.oracle_seq.argtypes = [I, I, I, I, P, P, P, P, I]
    lib.oracle_newton.argtypes = [I, I, I, I, I, P, P, P, P, P, P, I]
    lib.oracle_adjoint.argtypes = [I, I, I, I, P, P, P, P, P, P, P, P, I]
    lib.oracle_cell.argtypes = [I, I, P, P, P, P, P, P, P]
    lib.oracle_scan.argtypes = [I, I, I, I, P, P, P, P, I]
    lib.oracle_scan_dense.argtypes = [I, I, I, P, P, P, P, I]
    for f in (lib.oracle_seq, lib.oracle_newton, lib.oracle_adjoint, lib.oracle_cell, lib.oracle_scan,
              lib.oracle_scan_dense):
        f.restype = I
    return lib


def build_variant(source_text: str, out_path) -> Path:
    """Compile a modified copy of the oracle source (used only to check that the
    pins reject planted mistakes)."""
    out_path = Path(out_path)
    src = out_path.with_suffix(".c")
    src.write_text(source_text)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", str(out_path), str(src),
                    "-lm", "-lpthread"], check=True)
    return out_path


@contextlib.contextmanager
def using(path):
    """Temporarily route every call of this module to another build of the oracle."""
    global _lib
    saved = _lib
    _lib = _bind(path)
    try:
        yield
    finally:
        _lib = saved


def _load():
    global _lib
    if _lib is None:
        if not LIB.exists():
            build()
        _lib = _bind(LIB)
    return _lib


def default_threads() -> int:
    env = os.environ.get("OMP_NUM_THREADS")
    n = int(env) if env and env.isdigit() else (os.cpu_count() or 1)
    return max(1, min(n, os.cpu_count() or 1))


def _np(x, dtype):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor on the CPU
        x = x.detach().cpu()
        if str(x.dtype) == "torch.bfloat16":
            x = x.float()
        x = x.numpy()
    return np.ascontiguousarray(x, dtype=dtype)


def _ptr(x):
    return None if x is None else x.ctypes.data


def _shape(cell, u):
    B, L, G, D = u.shape
    if G != GATES[cell]:
        raise ValueError(f"{cell} expects {GATES[cell]} gates, u has {G}")
    return B, L, D


def seq(cell, u, a, s0=None, nthreads=None):
    """Sequential recurrence; returns states [NS][B][L][D]."""
    u = _np(u, np.float32)
    a = _np(a, np.float32)
    s0 = _np(s0, np.float64)
    B, L, D = _shape(cell, u)
    out = np.empty((NSTATE[cell], B, L, D), np.float64)
    rc = _load().oracle_seq(CELLS[cell], B, L, D, _ptr(u), _ptr(a), _ptr(s0), _ptr(out),
                            nthreads or default_threads())
    if rc:
        raise ValueError(f"oracle_seq failed ({rc})")
    return out


def newton(cell, u, a, K=3, s0=None, return_iterates=False, nthreads=None):
    """K Newton iterations from the zero sequence.

    Returns (states [NS][B][L][D], max_update [K][B]) and, when asked,
    all iterates [K][NS][B][L][D].
    """
    u = _np(u, np.float32)
    a = _np(a, np.float32)
    s0 = _np(s0, np.float64)
    B, L, D = _shape(cell, u)
    NS = NSTATE[cell]
    out = np.empty((NS, B, L, D), np.float64)
    upd = np.empty((K, B), np.float64)
    its = np.empty((K, NS, B, L, D), np.float64) if return_iterates else None
    rc = _load().oracle_newton(CELLS[cell], B, L, D, K, _ptr(u), _ptr(a), _ptr(s0), _ptr(out),
                               _ptr(upd), _ptr(its), nthreads or default_threads())
    if rc:
        raise ValueError(f"oracle_newton failed ({rc})")
    return (out, upd, its) if return_iterates else (out, upd)


def adjoint(cell, u, a, S, dh, s0=None, nthreads=None):
    """Adjoint along trajectory S [NS][B][L][D] for upstream dh [B][L][D].

    Returns (du [B][L][G][D], ds0 [NS][B][D], da [G][D]).
    """
    u = _np(u, np.float32)
    a = _np(a, np.float32)
    S = _np(S, np.float64)
    dh = _np(dh, np.float32)
    s0 = _np(s0, np.float64)
    B, L, D = _shape(cell, u)
    NS, G = NSTATE[cell], GATES[cell]
    if S.shape != (NS, B, L, D) or dh.shape != (B, L, D):
        raise ValueError("S must be [NS][B][L][D] and dh [B][L][D]")
    du = np.empty((B, L, G, D), np.float64)
    ds0 = np.empty((NS, B, D), np.float64)
    da = np.empty((G, D), np.float64)
    rc = _load().oracle_adjoint(CELLS[cell], B, L, D, _ptr(u), _ptr(a), _ptr(s0), _ptr(S),
                                _ptr(dh), _ptr(du), _ptr(ds0), _ptr(da),
                                nthreads or default_threads())
    if rc:
        raise ValueError(f"oracle_adjoint failed ({rc})")
    return du, ds0, da


def cell(cell_name, s, u, a):
    """Evaluate the cell on n channels: s [NS][n], u [G][n], a [G][n].

    Returns dict with f [NS][n], J [NS][NS][n], dfdu [NS][G][n], dfda [NS][G][n].
    """
    s = _np(s, np.float64)
    u = _np(u, np.float64)
    a = _np(a, np.float64)
    NS, G = NSTATE[cell_name], GATES[cell_name]
    n = s.shape[-1]
    if s.shape != (NS, n) or u.shape != (G, n) or a.shape != (G, n):
        raise ValueError("shapes must be s [NS][n], u [G][n], a [G][n]")
    f = np.empty((NS, n))
    J = np.empty((NS, NS, n))
    dfdu = np.empty((NS, G, n))
    dfda = np.empty((NS, G, n))
    rc = _load().oracle_cell(CELLS[cell_name], n, _ptr(s), _ptr(u), _ptr(a), _ptr(f), _ptr(J),
                             _ptr(dfdu), _ptr(dfda))
    if rc:
        raise ValueError(f"oracle_cell failed ({rc})")
    return dict(f=f, J=J, dfdu=dfdu, dfda=dfda)


def scan(A, b, s0=None, nthreads=None):
    """Linear recurrence s_l = A_l s_{l-1} + b_l per channel, s_{-1} = s0.

    ns = 1: A, b [B][L][D]; ns = 2: A [2][2][B][L][D] (block rows first), b
    [2][B][L][D]; s0 [ns][B][D] or None. Returns s with the shape of b (fp64).
    """
    A = _np(A, np.float64)
    b = _np(b, np.float64)
    if A.ndim == 3:
        ns, shape = 1, b.shape
    elif A.ndim == 5 and A.shape[:2] == (2, 2):
        ns, shape = 2, b.shape[1:]
    else:
        raise ValueError("A must be [B][L][D] or [2][2][B][L][D]")
    if b.shape != ((shape) if ns == 1 else (2,) + tuple(shape)) or A.shape[-3:] != tuple(shape):
        raise ValueError("A and b shapes disagree")
    B, L, D = shape
    s0 = _np(s0, np.float64)
    if s0 is not None and s0.shape != (ns, B, D):
        raise ValueError("s0 must be [ns][B][D]")
    s = np.empty(b.shape, np.float64)
    rc = _load().oracle_scan(ns, B, L, D, _ptr(A), _ptr(b), _ptr(s0), _ptr(s), nthreads or default_threads())
    if rc:
        raise ValueError(f"oracle_scan failed ({rc})")
    return s


def scan_dense(A, b, s0=None, nthreads=None):
    """Linear recurrence with a dense n x n matrix per step: A [B][L][n][n]
    (A_l[r][q] multiplies s_{l-1}[q] into s_l[r]), b [B][L][n], s0 [B][n] or
    None. Returns s [B][L][n] (fp64)."""
    A = _np(A, np.float64)
    b = _np(b, np.float64)
    if A.ndim != 4 or A.shape[2] != A.shape[3] or b.shape != A.shape[:3]:
        raise ValueError("A must be [B][L][n][n] and b [B][L][n]")
    B, L, n = b.shape
    s0 = _np(s0, np.float64)
    if s0 is not None and s0.shape != (B, n):
        raise ValueError("s0 must be [B][n]")
    s = np.empty(b.shape, np.float64)
    rc = _load().oracle_scan_dense(B, L, n, _ptr(A), _ptr(b), _ptr(s0), _ptr(s), nthreads or default_threads())
    if rc:
        raise ValueError(f"oracle_scan_dense failed ({rc})")
    return s


def flags(max_update, tol=1e-4, early_exit=False):
    """Iteration count and per-row convergence flags from the update sizes.

    converged[b] = max_update[iters-1][b] <= tol. Without early exit iters = K;
    with it, iters is the first k whose rows all satisfy the test (else K).
    """
    upd = np.asarray(max_update, np.float64)
    K = upd.shape[0]
    iters = K
    if early_exit:
        for k in range(K):
            if np.all(upd[k] <= tol):
                iters = k + 1
                break
    conv = (upd[iters - 1] <= tol).astype(np.int32)
    return iters, conv
