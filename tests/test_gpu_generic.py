"""Generic-cell tier (user cell in torch, Jacobian by forward-mode AD, linear
system by the library's scan) on the GPU: the GRU and LSTM written as user
cells reproduce the oracle's Newton iterate and the fused kernels; a cell the
library has no kernel for reproduces its own sequential recurrence."""
import numpy as np
import pytest
import torch

from nonlinear_rnn_solve_newton_amd import binding, generic
from nonlinear_rnn_solve_newton_amd.workloads import make_inputs
from oracle import oracle as O
from tests.helpers import STATE_TOL, assert_close, say

pytestmark = pytest.mark.gpu

SHAPES = [(1, 1, 1), (2, 3, 5), (1, 129, 64), (2, 1000, 96), (3, 700, 130)]


@pytest.mark.parametrize("cell", ["gru", "lstm"])
@pytest.mark.parametrize("B,L,D", SHAPES, ids=[f"{b}x{l}x{d}" for b, l, d in SHAPES])
def test_generic_tier_matches_oracle_and_fused(cell, B, L, D):
    say(f"generic {cell} B={B} L={L} D={D}")
    x = make_inputs(cell, B, L, D, seed=3000 + B + L + D, u_dtype="bf16")
    dev = torch.device("cuda:0")
    u, a = x.u.to(dev), x.a.to(dev)
    if cell == "gru":
        S = generic.newton_solve(lambda h, uu: generic.gru_step(h, uu, a), u, B=B, L=L, D=D, iters=3)
        got = S[None]
    else:
        S = generic.newton_solve(lambda s, uu: generic.lstm_step(s, uu, a), u, B=B, L=L, D=D, iters=3,
                                 block=2)
        got = S
    torch.cuda.synchronize()
    got = got.cpu().double().numpy()
    want, _ = O.newton(cell, x.u, x.a, K=3)
    assert_close(got, want, STATE_TOL, f"generic {cell} vs oracle")
    r = binding.solve(cell, u, a, iters=3)
    fused = np.stack([t.cpu().double().numpy() for t in ([r["h"]] if cell == "gru" else [r["c"], r["h"]])])
    assert_close(got, fused, 2 * STATE_TOL, f"generic {cell} vs fused")


def _tanh_rnn_sequential(u, a, w, s0):
    """s_l = tanh(a * s_{l-1} + w * s_{l-1}^2 / (1 + s_{l-1}^2) + u_l), fp64, by a loop."""
    B, L, D = u.shape
    s = s0.clone()
    out = torch.empty(B, L, D, dtype=torch.float64)
    for l in range(L):
        s = torch.tanh(a * s + w * s * s / (1 + s * s) + u[:, l])
        out[:, l] = s
    return out


def test_generic_tier_on_a_cell_without_a_kernel():
    """A diagonal cell the library does not implement: after K iterations the
    first K rows are the sequential recurrence (the residual Jacobian is unit
    lower-bidiagonal), and iterating to the fixed point gives all of it."""
    say("generic custom cell")
    B, L, D = 2, 300, 48
    g = torch.Generator().manual_seed(61)
    u = torch.randn(B, L, D, generator=g)
    a = 0.9 * (2 * torch.rand(D, generator=g) - 1)
    w = 0.5 * torch.rand(D, generator=g)
    s0 = torch.randn(B, D, generator=g)
    want = _tanh_rnn_sequential(u.double(), a.double(), w.double(), s0.double()).numpy()
    dev = torch.device("cuda:0")
    ud, ad, wd, s0d = u.to(dev), a.to(dev), w.to(dev), s0.to(dev)
    step = lambda s, uu: torch.tanh(ad * s + wd * s * s / (1 + s * s) + uu)  # noqa: E731
    S3 = generic.newton_solve(step, ud, s0d, B=B, L=L, D=D, iters=3).cpu().double().numpy()
    assert_close(S3[:, :3], want[:, :3], 1e-5, "rows l < K after K iterations")
    S, upd = generic.newton_solve(step, ud, s0d, B=B, L=L, D=D, iters=12, return_updates=True)
    assert upd[-1] < 1e-5 and upd[-1] < upd[2]
    assert_close(S.cpu().double().numpy(), want, STATE_TOL, "fixed point vs sequential")


def _elman_dense_newton_numpy(u, W, s0, K):
    """Newton on F_l(S) = S_l - tanh(W S_{l-1} + u_l) for one row, each step a
    dense (L n) x (L n) solve (numpy.linalg.solve), from S = 0."""
    L, n = u.shape
    S = np.zeros((L, n))
    for _ in range(K):
        P = np.vstack([s0[None], S[:-1]])
        f = np.tanh(P @ W.T + u)
        F = (S - f).reshape(-1)
        J = np.eye(L * n)
        for l in range(1, L):
            J[l * n:(l + 1) * n, (l - 1) * n:l * n] = -(1 - f[l] ** 2)[:, None] * W
        S = S - np.linalg.solve(J, F).reshape(L, n)
    return S


@pytest.mark.parametrize("n", [4, 32])
def test_generic_dense_elman_matches_dense_newton(n):
    """A dense-Jacobian RNN (h' = tanh(W h + u), W dense) through the generic
    tier and pararnn_scan_dense: each Newton iterate equals the same iteration
    with the whole system solved densely."""
    say(f"generic dense Elman n={n}")
    B, L = 2, 40
    g = torch.Generator().manual_seed(90 + n)
    W = 0.9 * torch.linalg.qr(torch.randn(n, n, generator=g, dtype=torch.float64))[0]
    u = torch.randn(B, L, n, generator=g)
    s0 = torch.randn(B, n, generator=g)
    dev = torch.device("cuda:0")
    Wd = W.float().to(dev)
    step = lambda h, uu: torch.tanh(h @ Wd.T + uu)  # noqa: E731
    for K in (1, 3):
        S = generic.newton_solve(step, u.to(dev), s0.to(dev), B=B, L=L, D=n, iters=K, block="dense")
        got = S.cpu().double().numpy()
        want = np.stack([_elman_dense_newton_numpy(u[b].double().numpy(), W.numpy(), s0[b].double().numpy(), K)
                         for b in range(B)])
        assert_close(got, want, STATE_TOL, f"dense Elman K={K}")


def test_generic_dense_elman_fixed_point():
    """Iterated to convergence the dense tier reproduces the sequential recurrence."""
    B, L, n = 3, 500, 16
    g = torch.Generator().manual_seed(93)
    W = 0.8 * torch.linalg.qr(torch.randn(n, n, generator=g, dtype=torch.float64))[0]
    u = torch.randn(B, L, n, generator=g)
    want = torch.empty(B, L, n, dtype=torch.float64)
    h = torch.zeros(B, n, dtype=torch.float64)
    for l in range(L):
        h = torch.tanh(h @ W.T + u[:, l].double())
        want[:, l] = h
    dev = torch.device("cuda:0")
    Wd = W.float().to(dev)
    S, upd = generic.newton_solve(lambda hh, uu: torch.tanh(hh @ Wd.T + uu), u.to(dev), B=B, L=L, D=n, iters=12,
                                  block="dense", return_updates=True)
    assert upd[-1] < 1e-5
    assert_close(S.cpu().double().numpy(), want.numpy(), STATE_TOL, "dense fixed point vs sequential")
