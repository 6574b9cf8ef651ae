"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
binding and the fp64 oracle on the same seeded inputs, and compare."""
from __future__ import annotations

import sys

import numpy as np
import torch

from nonlinear_rnn_solve_newton_amd import binding
from nonlinear_rnn_solve_newton_amd.workloads import gather_channels
from oracle import oracle as O

STATE_TOL = 1e-4  # max-abs error allowed on the fp32 states after K Newton iterations
FLAG_MARGIN_ABS = 2e-5  # flags are compared only where |update - tol| exceeds this margin


def say(*msg):
    print(*msg, file=sys.stderr, flush=True)


def dev():
    return torch.device("cuda:0")


def gpu_solve(cell, x, iters=3, s0=None, tol=1e-4, early_exit=False, u=None, a=None, schedule="auto"):
    """Run the HIP solve on the inputs of x (u or a replaced when given); returns
    (states [NS][B][L][D] fp64, iters, conv, max_update)."""
    d = dev()
    ug = (x.u if u is None else u).to(d)
    ag = (x.a if a is None else a).to(d)
    kw = {}
    if s0 is not None:
        s0t = torch.as_tensor(s0, dtype=torch.float32)
        if cell == "gru":
            kw["h0"] = s0t[0].contiguous().to(d)
        else:
            kw["c0"] = s0t[0].contiguous().to(d)
            kw["h0"] = s0t[1].contiguous().to(d)
    r = binding.solve(cell, ug, ag, iters=iters, tol=tol, early_exit=early_exit, schedule=schedule, **kw)
    torch.cuda.synchronize()
    st = [r["h"]] if cell == "gru" else [r["c"], r["h"]]
    S = np.stack([t.cpu().double().numpy() for t in st])
    return S, int(r["iters"].item()), r["converged"].cpu().numpy(), r["max_update"].cpu().double().numpy()


def s0_float32(s0):
    """Initial states as the GPU sees them (rounded to fp32)."""
    return None if s0 is None else np.asarray(s0, np.float32).astype(np.float64)


def assert_close(got, want, tol, what):
    err = np.abs(got - want)
    bad = ~(err <= tol)  # NaN counts as bad
    if bad.any():
        idx = np.unravel_index(np.argmax(np.where(np.isnan(err), np.inf, err)), err.shape)
        raise AssertionError(f"{what}: max |err| = {np.nanmax(err):.3e} > {tol:g} at {idx}: "
                             f"got {got[idx]!r} want {want[idx]!r} ({int(bad.sum())} bad of {err.size})")
    return float(err.max()) if err.size else 0.0


def check_flags(iters, conv, oracle_upd, K, tol, early_exit=False):
    """Bit-exact flags where the oracle's update is clear of tol by the margin;
    returns the number of rows that were ambiguous (skipped)."""
    want_iters, want_conv = O.flags(oracle_upd, tol, early_exit)
    margin = max(FLAG_MARGIN_ABS, 0.1 * tol)
    ambiguous_rows = np.zeros(oracle_upd.shape[1], bool)
    for k in range(oracle_upd.shape[0]):
        ambiguous_rows |= np.abs(oracle_upd[k] - tol) <= margin
    if not early_exit or not ambiguous_rows.any():
        assert iters == want_iters, f"iters {iters} != oracle {want_iters}"
    ok = ~ambiguous_rows
    assert np.array_equal(conv[ok], want_conv[ok]), f"converged {conv} != oracle {want_conv}"
    return int(ambiguous_rows.sum())


def sampled_oracle(cell, x, chans, iters=3):
    """Oracle Newton iterate on a gathered subset of channels (full L)."""
    D = x.u.shape[-1]
    u = gather_channels(x.u, chans, D)          # [1][L][G][n]
    a = x.a[:, (chans % D)].contiguous()         # [G][n]
    return O.newton(cell, u, a, K=iters)


def pick(S, chans, D):
    """S [NS][B][L][D] -> [NS][1][L][n] at the given channels."""
    b = (chans // D).numpy()
    d = (chans % D).numpy()
    return np.stack([S[:, bi, :, di] for bi, di in zip(b, d)], axis=-1)[:, None]
