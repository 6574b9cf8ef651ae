"""GPU parity of the adjoint (reverse scan) against the fp64 oracle's BPTT.

Two forms: same-state (the oracle's fp64 trajectory, rounded to fp32, is fed to
the GPU adjoint) and end-to-end (GPU forward then GPU adjoint, against the
oracle's Newton iterate then the oracle's adjoint)."""
import numpy as np
import pytest
import torch

from nonlinear_rnn_solve_newton_amd import binding
from nonlinear_rnn_solve_newton_amd.workloads import make_inputs
from oracle import oracle as O
from tests.helpers import assert_close, say

pytestmark = pytest.mark.gpu

GRAD_TOL = 1e-4

SHAPES = [(1, 1, 1), (1, 2, 3), (2, 5, 64), (1, 63, 65), (2, 127, 6), (1, 129, 128),
          (3, 1000, 64), (2, 1000, 200), (1, 4097, 3), (2, 300, 1000)]


def _gpu_adjoint(cell, x, S, s0=None, want_ds0=True, want_da=True):
    d = torch.device("cuda:0")
    kw = {}
    if cell == "lstm":
        kw["c"] = torch.as_tensor(S[0], dtype=torch.float32).contiguous().to(d)
    h = torch.as_tensor(S[-1], dtype=torch.float32).contiguous().to(d)
    if s0 is not None:
        s0t = torch.as_tensor(s0, dtype=torch.float32)
        kw["h0"] = s0t[-1].contiguous().to(d)
        if cell == "lstm":
            kw["c0"] = s0t[0].contiguous().to(d)
    r = binding.adjoint(cell, x.u.to(d), x.a.to(d), h, x.dh.to(d), want_ds0=want_ds0, want_da=want_da, **kw)
    torch.cuda.synchronize()
    out = {k: (v.cpu().double().numpy() if isinstance(v, torch.Tensor) else v) for k, v in r.items() if k != "ws"}
    return out


@pytest.mark.parametrize("cell", ["gru", "lstm"])
@pytest.mark.parametrize("u_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,L,D", SHAPES, ids=[f"{b}x{l}x{d}" for b, l, d in SHAPES])
def test_adjoint_same_state(cell, u_dtype, B, L, D):
    say(f"adjoint {cell} {u_dtype} B={B} L={L} D={D}")
    x = make_inputs(cell, B, L, D, seed=2000 + B + L + D, u_dtype=u_dtype, adjoint=True)
    S, _ = O.newton(cell, x.u, x.a, K=3)
    S32 = S.astype(np.float32).astype(np.float64)  # the GPU reads the trajectory in fp32
    du, ds0, da = O.adjoint(cell, x.u, x.a, S32, x.dh)
    g = _gpu_adjoint(cell, x, S32)
    assert_close(g["du"], du, GRAD_TOL, "du")
    assert_close(g["ds0"], ds0, GRAD_TOL, "ds0")
    # da sums B*L terms: compare relative to the size of the sum
    scale = max(1.0, float(np.abs(da).max()))
    assert_close(g["da"], da, GRAD_TOL * scale, "da")


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_adjoint_whole_chunks(cell):
    """L a whole number of the launch's chunks and D of its channel tiles:
    every workgroup, the last chunk's included, runs the unmasked full-tile
    path, whose lanes read the state row before their first step from the
    neighbouring lane's rows and the previous chunk."""
    B = 2
    pl = binding.plan(cell, binding.OP_ADJOINT, B, 1000, 256)
    L, D = 3 * pl["chunk"], 2 * pl["channels"]
    say(f"adjoint {cell} B={B} L={L} D={D} (whole chunks of {pl['chunk']} steps, {pl['channels']} channels)")
    x = make_inputs(cell, B, L, D, seed=2500 + L, u_dtype="bf16", adjoint=True)
    S, _ = O.newton(cell, x.u, x.a, K=3)
    S32 = S.astype(np.float32).astype(np.float64)
    du, ds0, da = O.adjoint(cell, x.u, x.a, S32, x.dh)
    g = _gpu_adjoint(cell, x, S32)
    assert_close(g["du"], du, GRAD_TOL, "du")
    assert_close(g["ds0"], ds0, GRAD_TOL, "ds0")
    scale = max(1.0, float(np.abs(da).max()))
    assert_close(g["da"], da, GRAD_TOL * scale, "da")


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_adjoint_end_to_end(cell):
    say(f"adjoint {cell} end to end")
    B, L, D = 2, 2000, 128
    x = make_inputs(cell, B, L, D, seed=41, u_dtype="bf16", adjoint=True)
    d = torch.device("cuda:0")
    r = binding.solve(cell, x.u.to(d), x.a.to(d), iters=3)
    g = binding.adjoint(cell, x.u.to(d), x.a.to(d), r["h"], x.dh.to(d), c=r.get("c"))
    torch.cuda.synchronize()
    S, _ = O.newton(cell, x.u, x.a, K=3)
    du, _, _ = O.adjoint(cell, x.u, x.a, S, x.dh)
    assert_close(g["du"].cpu().double().numpy(), du, GRAD_TOL, "du end to end")


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_adjoint_with_initial_state(cell):
    say(f"adjoint {cell} with initial state")
    B, L, D = 2, 500, 64
    x = make_inputs(cell, B, L, D, seed=43, u_dtype="bf16", adjoint=True)
    NS = 2 if cell == "lstm" else 1
    s0 = np.random.default_rng(4).normal(size=(NS, B, D)).astype(np.float32).astype(np.float64)
    S = O.seq(cell, x.u, x.a, s0=s0).astype(np.float32).astype(np.float64)
    du, ds0, da = O.adjoint(cell, x.u, x.a, S, x.dh, s0=s0)
    g = _gpu_adjoint(cell, x, S, s0=s0)
    assert_close(g["du"], du, GRAD_TOL, "du")
    assert_close(g["ds0"], ds0, GRAD_TOL, "ds0")


def test_adjoint_repeat():
    """A second adjoint in the same workspace reproduces the first, to
    rounding (the look-back's association may vary; the da reduction order is
    fixed)."""
    say("adjoint lstm repeat")
    x = make_inputs("lstm", 2, 3000, 128, seed=47, u_dtype="bf16", adjoint=True)
    d = torch.device("cuda:0")
    r = binding.solve("lstm", x.u.to(d), x.a.to(d))
    g1 = binding.adjoint("lstm", x.u.to(d), x.a.to(d), r["h"], x.dh.to(d), c=r["c"], want_da=True)
    du1, da1 = g1["du"].clone(), g1["da"].clone()
    g2 = binding.adjoint("lstm", x.u.to(d), x.a.to(d), r["h"], x.dh.to(d), c=r["c"], want_da=True,
                         ws=g1["ws"])
    torch.cuda.synchronize()
    assert float((du1 - g2["du"]).abs().max()) <= 1e-6
    assert float((da1 - g2["da"]).abs().max()) <= 1e-6 * max(1.0, float(da1.abs().max()))
