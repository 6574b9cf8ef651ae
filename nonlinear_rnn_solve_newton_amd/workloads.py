"""Seeded synthetic inputs for the ParaGRU / ParaLSTM Newton solve.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic. Both sides of every parity check (the HIP path and the
fp64 oracle) consume the tensors it returns, so they see identical bits.

Layouts (shared by the C-ABI and the oracle):
  u  : [B][L][G][D]  gate pre-activation inputs; GRU gates (z, r, c), LSTM gates
                     (i, f, o, g); fp32, or bf16 rounded to nearest even.
  a  : [G][D] fp32   diagonal recurrent coefficients, shared over B and L.
  dh : [B][L][D] fp32 upstream gradient dL/dh (adjoint workloads only).

Recipe: one CPU torch generator per workload, seeded with the workload's seed;
draw a = amax * (2 * U[0,1) - 1), then u ~ N(0, 1), then (adjoint only)
dh ~ N(0, 1), in that order. For the LSTM the forget-gate column gets +1 in
fp32 before any bf16 rounding. Channels are i.i.d.; a is per channel.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import torch

GATES = {"gru": 3, "lstm": 4}
NSTATE = {"gru": 1, "lstm": 2}
LSTM_FORGET_GATE = 1  # gate order (i, f, o, g)


@dataclass(frozen=True)
class Workload:
    name: str
    cell: str  # "gru" | "lstm"
    B: int
    L: int
    D: int
    u_dtype: str  # "f32" | "bf16"
    seed: int
    amax: float = 1.0
    forget_bias: float = 0.0
    adjoint: bool = False
    iters: int = 3

    @property
    def G(self) -> int:
        return GATES[self.cell]

    @property
    def NS(self) -> int:
        return NSTATE[self.cell]

    @property
    def N(self) -> int:
        return self.B * self.L * self.D


# The five workloads the throughput metric and the parity suite are defined on.
WORKLOADS = {
    w.name: w
    for w in [
        Workload("gru_b1_l1024_d64_f32", "gru", 1, 1024, 64, "f32", seed=0),
        Workload("gru_b8_l4096_d1024_bf16", "gru", 8, 4096, 1024, "bf16", seed=1),
        Workload("lstm_b8_l4096_d1024_bf16", "lstm", 8, 4096, 1024, "bf16", seed=2,
                 forget_bias=1.0),
        Workload("gru_b1_l65536_d2048_bf16", "gru", 1, 65536, 2048, "bf16", seed=3,
                 amax=0.9),
        Workload("lstm_b16_l2048_d4096_bf16_adjoint", "lstm", 16, 2048, 4096, "bf16",
                 seed=4, adjoint=True),
    ]
}

# The workload the headline throughput number is quoted on: the largest one
# (the 7B-layer-shaped ParaLSTM, forward solve plus adjoint).
HEADLINE = "lstm_b16_l2048_d4096_bf16_adjoint"


@dataclass
class Inputs:
    u: torch.Tensor  # [B][L][G][D], fp32 or bf16, CPU
    a: torch.Tensor  # [G][D] fp32, CPU
    dh: Optional[torch.Tensor] = None  # [B][L][D] fp32, CPU
    meta: dict = field(default_factory=dict)


def make_inputs(cell: str, B: int, L: int, D: int, *, seed: int, u_dtype: str = "bf16",
                amax: float = 1.0, forget_bias: Optional[float] = None,
                adjoint: bool = False, a_zero: bool = False) -> Inputs:
    """Draw one seeded input set (see the module docstring for the recipe).

    forget_bias defaults to +1 for the LSTM and 0 for the GRU. a_zero replaces
    the recurrent coefficients by zeros after drawing them (the draw order, and
    so u and dh, stay the same), which is the linear-cell special case.
    """
    G = GATES[cell]
    if forget_bias is None:
        forget_bias = 1.0 if cell == "lstm" else 0.0
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    a = amax * (2.0 * torch.rand(G, D, generator=g, dtype=torch.float32) - 1.0)
    u = torch.randn(B, L, G, D, generator=g, dtype=torch.float32)
    if cell == "lstm" and forget_bias != 0.0:
        u[:, :, LSTM_FORGET_GATE, :] += forget_bias
    if u_dtype == "bf16":
        u = u.to(torch.bfloat16)
    elif u_dtype != "f32":
        raise ValueError(f"u_dtype must be 'f32' or 'bf16', got {u_dtype!r}")
    dh = torch.randn(B, L, D, generator=g, dtype=torch.float32) if adjoint else None
    if a_zero:
        a = torch.zeros_like(a)
    return Inputs(u=u.contiguous(), a=a.contiguous(), dh=dh,
                  meta=dict(cell=cell, B=B, L=L, D=D, seed=seed, u_dtype=u_dtype))


def workload_inputs(w: Workload) -> Inputs:
    return make_inputs(w.cell, w.B, w.L, w.D, seed=w.seed, u_dtype=w.u_dtype, amax=w.amax,
                       forget_bias=w.forget_bias, adjoint=w.adjoint)


def sample_channels(B: int, D: int, n: int, seed: int = 1234) -> torch.Tensor:
    """n distinct (b, d) channel ids b*D + d, sorted, drawn with their own seed."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    n = min(n, B * D)
    return torch.randperm(B * D, generator=g)[:n].sort().values


def gather_channels(x: torch.Tensor, chans: torch.Tensor, D: int) -> torch.Tensor:
    """Pick channels out of a [B][L][..][D] tensor into a [1][L][..][n] tensor.

    Channels of the diagonal cells never interact, so a gathered sub-problem is
    solved exactly like the same channels inside the full problem.
    """
    b = (chans // D).tolist()
    d = (chans % D).tolist()
    cols = [x[bi, ..., di] for bi, di in zip(b, d)]  # each [L] or [L][G]
    return torch.stack(cols, dim=-1).unsqueeze(0).contiguous()


# ---------------------------------------------------------------------------
# The linear scan alone. Coefficients drawn so the recurrence stays bounded:
# A ~ U(-amax, amax) per channel and step (2x2 blocks: each entry
# U(-amax/2, amax/2), so every row of a block sums to at most amax in
# magnitude), b ~ N(0, 1), s0 ~ N(0, 1); drawn in that order.

@dataclass(frozen=True)
class ScanWorkload:
    name: str
    ns: int  # 1: diagonal, 2: 2x2 blocks
    B: int
    L: int
    D: int
    seed: int
    amax: float = 0.95

    @property
    def N(self) -> int:
        return self.B * self.L * self.D


SCAN_WORKLOADS = {
    w.name: w
    for w in [
        ScanWorkload("scan_diag_b8_l4096_d1024", 1, 8, 4096, 1024, seed=5),
        ScanWorkload("scan_block2_b8_l4096_d1024", 2, 8, 4096, 1024, seed=6),
    ]
}


@dataclass
class ScanInputs:
    A: torch.Tensor  # [B][L][D] or [2][2][B][L][D] fp32, CPU
    b: torch.Tensor  # [B][L][D] or [2][B][L][D] fp32, CPU
    s0: torch.Tensor  # [B][D] or [2][B][D] fp32, CPU


def make_scan_inputs(ns: int, B: int, L: int, D: int, *, seed: int, amax: float = 0.95) -> ScanInputs:
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    if ns == 1:
        A = amax * (2.0 * torch.rand(B, L, D, generator=g, dtype=torch.float32) - 1.0)
        b = torch.randn(B, L, D, generator=g, dtype=torch.float32)
        s0 = torch.randn(B, D, generator=g, dtype=torch.float32)
    elif ns == 2:
        A = 0.5 * amax * (2.0 * torch.rand(2, 2, B, L, D, generator=g, dtype=torch.float32) - 1.0)
        b = torch.randn(2, B, L, D, generator=g, dtype=torch.float32)
        s0 = torch.randn(2, B, D, generator=g, dtype=torch.float32)
    else:
        raise ValueError("ns must be 1 or 2")
    return ScanInputs(A=A.contiguous(), b=b.contiguous(), s0=s0.contiguous())


def scan_workload_inputs(w: ScanWorkload) -> ScanInputs:
    return make_scan_inputs(w.ns, w.B, w.L, w.D, seed=w.seed, amax=w.amax)


# ---------------------------------------------------------------------------
# Dense recurrence (n x n matrix per step): A_l = 0.95 Q_l with Q_l a random
# orthogonal matrix (QR of a Gaussian matrix, signs fixed by diag(R) > 0), so
# every step contracts by exactly 0.95 in the 2-norm; then b ~ N(0, 1),
# s0 ~ N(0, 1), drawn in that order.

@dataclass(frozen=True)
class DenseScanWorkload:
    name: str
    B: int
    L: int
    n: int
    seed: int
    scale: float = 0.95

    @property
    def N(self) -> int:
        return self.B * self.L * self.n


DENSE_WORKLOADS = {
    w.name: w
    for w in [
        DenseScanWorkload("scan_dense_b8_l4096_n32", 8, 4096, 32, seed=7),
    ]
}


@dataclass
class DenseScanInputs:
    A: torch.Tensor   # [B][L][n][n] fp32, CPU
    b: torch.Tensor   # [B][L][n]
    s0: torch.Tensor  # [B][n]


def make_dense_scan_inputs(B: int, L: int, n: int, *, seed: int, scale: float = 0.95) -> DenseScanInputs:
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    M = torch.randn(B, L, n, n, generator=g, dtype=torch.float64)
    Q, R = torch.linalg.qr(M)
    Q = Q * torch.sign(torch.diagonal(R, dim1=-2, dim2=-1)).unsqueeze(-2)
    A = (scale * Q).to(torch.float32)
    b = torch.randn(B, L, n, generator=g, dtype=torch.float32)
    s0 = torch.randn(B, n, generator=g, dtype=torch.float32)
    return DenseScanInputs(A=A.contiguous(), b=b.contiguous(), s0=s0.contiguous())


def dense_workload_inputs(w: DenseScanWorkload) -> DenseScanInputs:
    return make_dense_scan_inputs(w.B, w.L, w.n, seed=w.seed, scale=w.scale)
