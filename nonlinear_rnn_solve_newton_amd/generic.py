"""Generic-cell tier: Newton solve of a user-written recurrence whose Jacobian
is diagonal or 2x2 block-diagonal per channel, with the linear system of each
iteration solved by the library's scan (pararnn_scan_diag /
pararnn_scan_block2).

The ParaRNN article (cafecomtech.com, section "Como usar") has the user supply
a cell's one-step recurrence and leaves Newton, Jacobian assembly and the
parallel reduction to the framework; section "Engenharia pra escalar" requires
the cell's Jacobian to be diagonal or 2x2 block-diagonal. Here the user's
`step` is plain torch code, evaluated for all steps at once; its Jacobian
coefficients come from forward-mode AD (torch.func.jvp with unit tangents,
which for a diagonal Jacobian yields exactly its diagonal, and for 2x2 blocks
one block column per tangent). Each iteration then solves
    S_l = A_l S_{l-1} + (f_l - A_l P_l),   P_l = S^(k-1)_{l-1} (s0 at l = 0),
on the GPU. The fused cells of this library (GRU, LSTM) do all of this in one
kernel per iteration; this tier trades that for arbitrary cells.
"""
from __future__ import annotations

from typing import Callable, Optional

import torch

from . import binding


def _shift(S: torch.Tensor, s0: Optional[torch.Tensor], l_axis: int) -> torch.Tensor:
    """P_l = S_{l-1}, with s0 (or zero) at l = 0, along axis l_axis."""
    first = torch.zeros_like(S.narrow(l_axis, 0, 1)) if s0 is None else s0.unsqueeze(l_axis)
    return torch.cat([first, S.narrow(l_axis, 0, S.shape[l_axis] - 1)], dim=l_axis)


def newton_solve(step: Callable, x, s0: Optional[torch.Tensor] = None, *, B: int, L: int, D: int,
                 iters: int = 3, block: int = 1, return_updates: bool = False):
    """Solve s_l = step(s_{l-1}, x_l) for l = 0..L-1 by `iters` Newton iterations
    from the zero sequence.

    block = 1: the state is one [B][L][D] tensor; step(P, x) -> f, elementwise
               per channel (its Jacobian must be diagonal).
    block = 2: the state is a pair of components, stacked [2][B][L][D];
               step(P, x) -> f with P and f of that shape (2x2 Jacobian blocks
               per channel).
    block = "dense": the state is [B][L][D] with D <= 32 and a dense D x D
               Jacobian per step (a generic RNN, ParaRNN article section
               "Engenharia pra escalar": n^2 storage, n^3 products); its D
               columns come from D tangents, and the linear system is solved by
               pararnn_scan_dense.
    x is passed to step unchanged (e.g. precomputed gate inputs [B][L][G][D]).
    s0: [B][D] (block 1) or [2][B][D] (block 2) fp32, or None for zero.
    Returns the K-th iterate (and the per-iteration max |update| if asked).
    """
    if block not in (1, 2, "dense"):
        raise ValueError("block must be 1, 2 or 'dense'")
    dev = x.device if isinstance(x, torch.Tensor) else torch.device("cuda:0")
    shape = (2, B, L, D) if block == 2 else (B, L, D)
    l_axis = 2 if block == 2 else 1
    S = torch.zeros(shape, dtype=torch.float32, device=dev)
    ws = None
    updates = []
    fn = lambda p: step(p, x)  # noqa: E731
    for _ in range(iters):
        P = _shift(S, s0, l_axis)
        if block == "dense":
            cols = []
            for k in range(D):  # column k of every step's Jacobian
                e = torch.zeros_like(P)
                e[..., k] = 1.0
                f, ck = torch.func.jvp(fn, (P,), (e,))
                cols.append(ck)
            A = torch.stack(cols, dim=-1)  # [B][L][D][D], A[..., r, k] = df_r / ds_k
            b = f - (A @ P.unsqueeze(-1)).squeeze(-1)
            r = binding.scan_dense(A.contiguous().float(), b.contiguous().float(), s0, ws=ws)
            ws = r["ws"]
            if return_updates:
                updates.append(float((r["s"] - S).abs().max()))
            S = r["s"]
            continue
        if block == 1:
            f, A = torch.func.jvp(fn, (P,), (torch.ones_like(P),))
            b = f - A * P
        else:
            e0 = torch.zeros_like(P)
            e0[0] = 1.0
            e1 = torch.zeros_like(P)
            e1[1] = 1.0
            f, col0 = torch.func.jvp(fn, (P,), (e0,))
            _, col1 = torch.func.jvp(fn, (P,), (e1,))
            A = torch.stack([torch.stack([col0[0], col1[0]]), torch.stack([col0[1], col1[1]])])
            b = f - torch.stack([A[0, 0] * P[0] + A[0, 1] * P[1], A[1, 0] * P[0] + A[1, 1] * P[1]])
        r = binding.scan(A.contiguous().float(), b.contiguous().float(), s0, ws=ws)
        ws = r["ws"]
        if return_updates:
            updates.append(float((r["s"] - S).abs().max()))
        S = r["s"]
    return (S, updates) if return_updates else S


# Reference cells written as a user would, in torch (used by the tests and the
# benchmark to compare the generic tier with the fused kernels).

def gru_step(h: torch.Tensor, u: torch.Tensor, a: torch.Tensor) -> torch.Tensor:
    """ParaGRU, gates (z, r, c); h [B][L][D], u [B][L][3][D], a [3][D]."""
    z = torch.sigmoid(a[0] * h + u[:, :, 0])
    r = torch.sigmoid(a[1] * h + u[:, :, 1])
    c = torch.tanh(a[2] * (r * h) + u[:, :, 2])
    return (1.0 - z) * h + z * c


def lstm_step(s: torch.Tensor, u: torch.Tensor, a: torch.Tensor) -> torch.Tensor:
    """ParaLSTM, gates (i, f, o, g), state (c, h) stacked [2][B][L][D]; u [B][L][4][D]."""
    c, h = s[0], s[1]
    i = torch.sigmoid(a[0] * h + u[:, :, 0])
    f = torch.sigmoid(a[1] * h + u[:, :, 1])
    o = torch.sigmoid(a[2] * h + u[:, :, 2])
    g = torch.tanh(a[3] * h + u[:, :, 3])
    cn = f * c + i * g
    return torch.stack([cn, o * torch.tanh(cn)])
