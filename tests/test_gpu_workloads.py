"""Parity on the five full-size workloads, in the launch configuration the
benchmark times (binding defaults, K = 3).

Channels of the diagonal cells never interact, so the fp64 oracle solves a
seeded sample of channels (b, d) over the full sequence and those outputs are
compared element by element. Properties that hold at any size are checked on
every channel: after K Newton iterations the first K rows equal the sequential
recurrence, and a row whose sampled update already exceeds tol cannot be
flagged converged.
"""
import numpy as np
import pytest
import torch

from nonlinear_rnn_solve_newton_amd import binding
from nonlinear_rnn_solve_newton_amd.workloads import (WORKLOADS, gather_channels, sample_channels,
                                                      workload_inputs)
from oracle import oracle as O
from tests.helpers import STATE_TOL, assert_close, say

pytestmark = pytest.mark.gpu

NSAMPLE = 48


def _sampled(t, chans, D):
    """[B][L][D] device tensor -> [L][n] numpy at the sampled channels."""
    b = (chans // D).to(t.device)
    d = (chans % D).to(t.device)
    return t[b, :, d].T.cpu().double().numpy()


@pytest.mark.parametrize("schedule", ["fused", "per_iteration"])
@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_parity(name, schedule):
    w = WORKLOADS[name]
    say(f"workload {name} ({schedule}): generating inputs")
    x = workload_inputs(w)
    dev = torch.device("cuda:0")
    u, a = x.u.to(dev), x.a.to(dev)
    say(f"workload {name}: solve")
    r = binding.solve(w.cell, u, a, iters=w.iters, schedule=schedule)
    torch.cuda.synchronize()
    chans = sample_channels(w.B, w.D, NSAMPLE, seed=7)
    us = gather_channels(x.u, chans, w.D)
    asmp = x.a[:, chans % w.D].contiguous()
    want, upd, its = O.newton(w.cell, us, asmp, K=w.iters, return_iterates=True)
    states = [r["h"]] if w.cell == "gru" else [r["c"], r["h"]]
    got = np.stack([_sampled(t, chans, w.D) for t in states])[:, None]  # [NS][1][L][n]
    err = assert_close(got, want, STATE_TOL, f"{name} sampled state")
    say(f"workload {name}: sampled state max err {err:.2e}")

    # flags: iters = K; a row whose sampled channels already moved by more than
    # tol (with margin) in the last iteration is not converged, and the
    # reported row maximum bounds the sampled one
    assert int(r["iters"].item()) == w.iters
    conv = r["converged"].cpu().numpy()
    mu = r["max_update"].cpu().double().numpy()
    last = np.abs(its[-1] - its[-2]).max(axis=(0, 1, 2))  # per sampled channel
    rows = (chans // w.D).numpy()
    for b in np.unique(rows):
        sampled_max = float(last[rows == b].max())
        if sampled_max > 1.2e-4:
            assert conv[b] == 0, f"row {b} flagged converged with sampled update {sampled_max}"
        assert mu[-1, b] >= sampled_max - 1e-5

    # any size: rows l < K equal the sequential recurrence on every channel
    K = w.iters
    seq = O.seq(w.cell, x.u[:, :K], x.a)
    full = np.stack([t[:, :K].cpu().double().numpy() for t in states])
    assert_close(full, seq, 1e-5, f"{name} first {K} rows vs sequential")

    if w.adjoint:
        say(f"workload {name}: adjoint")
        dh = x.dh.to(dev)
        g = binding.adjoint(w.cell, u, a, r["h"], dh, c=r.get("c"))
        torch.cuda.synchronize()
        dhs = gather_channels(x.dh, chans, w.D)
        du_want, _, _ = O.adjoint(w.cell, us, asmp, want, dhs)  # oracle adjoint at its own iterate
        bidx = (chans // w.D).to(dev)
        didx = (chans % w.D).to(dev)
        du_got = g["du"][bidx, :, :, didx].permute(1, 2, 0).cpu().double().numpy()[None]
        gerr = assert_close(du_got, du_want, 1e-4, f"{name} sampled du")
        say(f"workload {name}: sampled du max err {gerr:.2e}")

        # da and ds0 at full size: da[:, d] sums over every row b and step l,
        # so the oracle solves all B rows of a few sampled channels d
        say(f"workload {name}: adjoint with da and ds0")
        g2 = binding.adjoint(w.cell, u, a, r["h"], dh, c=r.get("c"), want_ds0=True, want_da=True)
        torch.cuda.synchronize()
        dsel = sorted(np.random.default_rng(11).choice(w.D, 4, replace=False).tolist())
        chans2 = torch.tensor([b * w.D + d for d in dsel for b in range(w.B)])
        us2 = gather_channels(x.u, chans2, w.D)
        as2 = x.a[:, chans2 % w.D].contiguous()
        want2, _ = O.newton(w.cell, us2, as2, K=w.iters)
        _, ds0_want, da_cols = O.adjoint(w.cell, us2, as2, want2, gather_channels(x.dh, chans2, w.D))
        da_want = da_cols.reshape(da_cols.shape[0], len(dsel), w.B).sum(axis=2)  # [G][n_d]
        da_got = g2["da"][:, dsel].cpu().double().numpy()
        scale = max(1.0, float(np.abs(da_want).max()))
        assert_close(da_got, da_want, 1e-4 * scale, f"{name} da at sampled channels")
        ds0_got = g2["ds0"][:, :, dsel].permute(0, 2, 1).reshape(ds0_want.shape[0], 1, -1).cpu().double().numpy()
        assert_close(ds0_got, ds0_want, 1e-4, f"{name} ds0 at sampled channels")
        assert float((g2["du"] - g["du"]).abs().max()) <= 1e-6  # requesting da and ds0 leaves du as it was
