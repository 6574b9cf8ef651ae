"""Launch modes and numerical stress, through the C ABI against the fp64 oracle.

1. Every kernel family switches its chunk carry from the decoupled look-back
   to the inclusive-only mode (each chunk waits for its neighbour's inclusive
   carry) at a threshold of workgroups per chunk row. Shapes on both sides of
   each threshold, checked with pararnn_plan_query, are compared with the
   oracle on every element.
2. Inclusive-only launches compose the chunk carries in a fixed order, so a
   repeated call gives identical bits (torch.equal), in the same and in a
   fresh workspace.
3. Stress: a GRU with every coefficient 1 and the update gate nearly closed
   (Jacobians within 1e-5 of 1 over 65536 steps) stays finite and matches the
   oracle; a GRU whose first linearisation has Jacobians near 4.5 overflows
   fp32 in the Newton iterate, which shows as a non-finite row maximum and a
   row not converged, never as an error.
"""
import numpy as np
import pytest
import torch

from nonlinear_rnn_solve_newton_amd import binding
from nonlinear_rnn_solve_newton_amd.workloads import make_inputs, make_scan_inputs
from oracle import oracle as O
from tests.helpers import STATE_TOL, assert_close, check_flags, say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")

# (cell, schedule, B, L, D, inclusive_only expected)
SOLVE_MODES = [
    ("gru", "fused", 1, 700, 2048, 1), ("gru", "fused", 1, 2048, 1024, 0),
    # the GRU's small-problem shape (16-channel tiles), both carry modes
    ("gru", "fused", 1, 700, 1024, 1), ("gru", "fused", 1, 700, 512, 0),
    ("lstm", "fused", 1, 700, 2048, 1), ("lstm", "fused", 1, 700, 1024, 0),
    # the LSTM's small-problem shape (8-channel tiles), both carry modes
    ("lstm", "fused", 1, 600, 512, 1), ("lstm", "fused", 1, 1000, 256, 0),
    ("gru", "per_iteration", 2, 700, 4096, 1), ("gru", "per_iteration", 1, 700, 4096, 0),
    ("lstm", "per_iteration", 1, 700, 4096, 1), ("lstm", "per_iteration", 1, 700, 2048, 0),
]


def _plan_mode(cell, op, B, L, D, schedule="auto", u_dtype=binding.BF16):
    return binding.plan(cell, op, B, L, D, 3, u_dtype, schedule)["inclusive_only"]


def _states(cell, r):
    return [r["h"]] if cell == "gru" else [r["c"], r["h"]]


@pytest.mark.parametrize("cell,schedule,B,L,D,incl", SOLVE_MODES,
                         ids=[f"{c}-{s}-{b}x{l}x{d}" for c, s, b, l, d, _ in SOLVE_MODES])
def test_solve_modes_every_element(cell, schedule, B, L, D, incl):
    assert _plan_mode(cell, binding.OP_SOLVE, B, L, D, schedule) == incl
    say(f"solve {cell} {schedule} B={B} L={L} D={D} inclusive_only={incl}")
    x = make_inputs(cell, B, L, D, seed=3000 + B + L + D, u_dtype="bf16")
    r = binding.solve(cell, x.u.to(DEV), x.a.to(DEV), iters=3, schedule=schedule)
    torch.cuda.synchronize()
    got = np.stack([t.cpu().double().numpy() for t in _states(cell, r)])
    want, upd = O.newton(cell, x.u, x.a, K=3)
    assert_close(got, want, STATE_TOL, f"{cell} {schedule} state")
    assert_close(r["max_update"].cpu().double().numpy(), upd, 1e-4, "max_update")
    check_flags(int(r["iters"].item()), r["converged"].cpu().numpy(), upd, 3, 1e-4)


ADJ_MODES = [("gru", 2, 700, 4096, 1), ("gru", 1, 700, 4096, 0), ("lstm", 1, 700, 4096, 1),
             ("lstm", 1, 700, 2048, 0)]


@pytest.mark.parametrize("cell,B,L,D,incl", ADJ_MODES, ids=[f"{c}-{b}x{l}x{d}" for c, b, l, d, _ in ADJ_MODES])
def test_adjoint_modes_every_element(cell, B, L, D, incl):
    assert _plan_mode(cell, binding.OP_ADJOINT, B, L, D) == incl
    say(f"adjoint {cell} B={B} L={L} D={D} inclusive_only={incl}")
    x = make_inputs(cell, B, L, D, seed=3100 + B + L + D, u_dtype="bf16", adjoint=True)
    S, _ = O.newton(cell, x.u, x.a, K=3)
    S32 = S.astype(np.float32)
    kw = {"c": torch.from_numpy(S32[0]).to(DEV)} if cell == "lstm" else {}
    g = binding.adjoint(cell, x.u.to(DEV), x.a.to(DEV), torch.from_numpy(S32[-1]).to(DEV), x.dh.to(DEV),
                        want_ds0=True, want_da=True, **kw)
    torch.cuda.synchronize()
    du, ds0, da = O.adjoint(cell, x.u, x.a, S32.astype(np.float64), x.dh)
    assert_close(g["du"].cpu().double().numpy(), du, 1e-4, "du")
    assert_close(g["ds0"].cpu().double().numpy(), ds0, 1e-4, "ds0")
    assert_close(g["da"].cpu().double().numpy(), da, 1e-4 * max(1.0, float(np.abs(da).max())), "da")


SCAN_MODES = [(1, 8, 300, 1024, 1), (1, 4, 300, 1024, 0), (2, 4, 300, 1024, 1), (2, 2, 300, 1024, 0)]


@pytest.mark.parametrize("ns,B,L,D,incl", SCAN_MODES, ids=[f"ns{n}-{b}x{l}x{d}" for n, b, l, d, _ in SCAN_MODES])
def test_scan_modes_every_element(ns, B, L, D, incl):
    op = binding.OP_SCAN_DIAG if ns == 1 else binding.OP_SCAN_BLOCK2
    assert _plan_mode("gru", op, B, L, D) == incl
    say(f"scan ns={ns} B={B} L={L} D={D} inclusive_only={incl}")
    x = make_scan_inputs(ns, B, L, D, seed=3200 + ns + B)
    r = binding.scan(x.A.to(DEV), x.b.to(DEV), x.s0.to(DEV))
    torch.cuda.synchronize()
    want = O.scan(x.A, x.b, x.s0 if ns == 2 else x.s0[None])
    assert_close(r["s"].cpu().double().numpy(), want, STATE_TOL, f"scan ns={ns}")


# --- bitwise repeatability of inclusive-only launches ------------------------

@pytest.mark.parametrize("cell,schedule,B,L,D", [("gru", "fused", 2, 3000, 2048), ("lstm", "fused", 2, 3000, 2048),
                                                 ("gru", "per_iteration", 2, 3000, 4096),
                                                 ("lstm", "per_iteration", 1, 3000, 4096)])
def test_inclusive_only_solve_repeats_bitwise(cell, schedule, B, L, D):
    assert _plan_mode(cell, binding.OP_SOLVE, B, L, D, schedule) == 1
    say(f"solve {cell} {schedule} B={B} L={L} D={D}: repeat")
    x = make_inputs(cell, B, L, D, seed=3300 + B, u_dtype="bf16")
    u, a = x.u.to(DEV), x.a.to(DEV)
    r1 = binding.solve(cell, u, a, schedule=schedule)
    first = [t.clone() for t in _states(cell, r1)] + [r1["max_update"].clone()]
    for ws in (r1["ws"], None):  # the same workspace, then a fresh one
        r2 = binding.solve(cell, u, a, schedule=schedule, ws=ws)
        torch.cuda.synchronize()
        again = _states(cell, r2) + [r2["max_update"]]
        assert all(torch.equal(p, q) for p, q in zip(first, again)), "inclusive-only solve not bit-identical"


@pytest.mark.parametrize("cell,B,D", [("gru", 2, 4096), ("lstm", 1, 4096)])
def test_inclusive_only_adjoint_repeats_bitwise(cell, B, D):
    L = 3000
    assert _plan_mode(cell, binding.OP_ADJOINT, B, L, D) == 1
    say(f"adjoint {cell} B={B} L={L} D={D}: repeat")
    x = make_inputs(cell, B, L, D, seed=3400 + B, u_dtype="bf16", adjoint=True)
    u, a, dh = x.u.to(DEV), x.a.to(DEV), x.dh.to(DEV)
    r = binding.solve(cell, u, a)
    g1 = binding.adjoint(cell, u, a, r["h"], dh, c=r.get("c"), want_ds0=True, want_da=True)
    first = [g1[k].clone() for k in ("du", "ds0", "da")]
    for ws in (g1["ws"], None):
        g2 = binding.adjoint(cell, u, a, r["h"], dh, c=r.get("c"), want_ds0=True, want_da=True, ws=ws)
        torch.cuda.synchronize()
        assert all(torch.equal(p, g2[k]) for p, k in zip(first, ("du", "ds0", "da"))), \
            "inclusive-only adjoint not bit-identical"


@pytest.mark.parametrize("ns,B", [(1, 8), (2, 4)])
def test_inclusive_only_scan_repeats_bitwise(ns, B):
    L, D = 3000, 1024
    op = binding.OP_SCAN_DIAG if ns == 1 else binding.OP_SCAN_BLOCK2
    assert _plan_mode("gru", op, B, L, D) == 1
    say(f"scan ns={ns} B={B} L={L} D={D}: repeat")
    x = make_scan_inputs(ns, B, L, D, seed=3500 + ns)
    A, b, s0 = x.A.to(DEV), x.b.to(DEV), x.s0.to(DEV)
    r1 = binding.scan(A, b, s0)
    first = r1["s"].clone()
    for ws in (r1["ws"], None):
        r2 = binding.scan(A, b, s0, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(first, r2["s"]), "inclusive-only scan not bit-identical"


# --- stress -----------------------------------------------------------------

def test_gru_jacobian_near_one_over_long_sequence():
    """Every coefficient 1 and u_z = -12: the update gate is nearly closed, each
    step changes h by about 6e-6 and every Jacobian lies within 1e-5 of 1, over
    65536 steps. The long products of near-unit Jacobians stay finite and the
    iterate matches the oracle."""
    B, L, D = 1, 65536, 64
    say(f"stress gru a=1, u_z=-12, B={B} L={L} D={D}")
    x = make_inputs("gru", B, L, D, seed=3600, u_dtype="f32")
    u = x.u.clone()
    u[:, :, 0, :] = -12.0
    a = torch.ones_like(x.a)
    r = binding.solve("gru", u.to(DEV), a.to(DEV), iters=3)
    torch.cuda.synchronize()
    got = r["h"].cpu().double().numpy()[None]
    want, upd = O.newton("gru", u, a, K=3)
    assert np.isfinite(got).all()
    assert_close(got, want, STATE_TOL, "near-unit Jacobians")
    assert_close(r["max_update"].cpu().double().numpy(), upd, 1e-4, "max_update")
    check_flags(int(r["iters"].item()), r["converged"].cpu().numpy(), upd, 3, 1e-4)


def test_block2_scan_near_unit_products_over_long_sequence():
    """The 2x2 scan with the LSTM's Jacobian pattern at the edge of stability:
    A = [[1 - 2^-16, 0], [q, 0]] (eigenvalues 1 - 2^-16 and 0, exactly
    representable), q ~ U(0, 0.5), b ~ N(0, 1), over 65536 steps. The first
    component sums its inputs over all of them (a random walk up to a few
    hundred), so the chunk and lane aggregates are products of thousands of
    near-unit blocks. They stay finite, and every element matches the fp64
    scan to 1e-4 of its series' largest magnitude. That is the bar here, not
    1e-4 of each value: the scan's fp32 products of near-unit factors drop a
    term below half an ulp at every factor (a bias of about 2^-25 each) and
    the carry, some hundreds here, is multiplied by them at each of the 1024
    chunk hand-offs (measured: 4.6e-5 of the series' largest magnitude, where
    a sequential fp32 recurrence, which forms no products, is off by about
    1.6e-6 of it). An LSTM solve with a forget gate that close to 1 is limited
    by fp32 even before the scan: the gate's own rounding, about 6e-8, is 0.6%
    of its distance from 1."""
    B, L, D = 1, 65536, 64
    say(f"stress block2 scan, a = 1 - 2^-16, B={B} L={L} D={D} (plan {binding.plan('gru', binding.OP_SCAN_BLOCK2, B, L, D)})")
    g = torch.Generator().manual_seed(3700)
    A = torch.zeros(2, 2, B, L, D)
    A[0, 0] = 1.0 - 2.0 ** -16
    A[1, 0] = 0.5 * torch.rand(B, L, D, generator=g)
    bb = torch.randn(2, B, L, D, generator=g)
    r = binding.scan(A.to(DEV), bb.to(DEV))
    torch.cuda.synchronize()
    got = r["s"].cpu().double().numpy()
    want = O.scan(A, bb)
    assert np.isfinite(got).all() and np.abs(want).max() > 50
    scale = np.maximum(1.0, np.abs(want).max(axis=2, keepdims=True))  # per (component, row, channel) series
    rel = np.abs(got - want) / scale
    assert np.all(rel <= 1e-4), f"max error {rel.max():.2e} of the series' largest magnitude"


def test_gru_iterate_overflow_is_flagged_not_an_error():
    """a_c = 8, u_z = 0, u_r = 5, u_c = 0.1: at the zero iterate the residual
    is z c~ = 0.5 tanh(0.1), about 0.05, and every Jacobian is about
    0.5 + 0.5 * 8 * 0.99 = 4.4, so the first Newton update grows like 4.4^l and
    passes the fp32 range near l = 62 (the fp64 oracle, with its wider range,
    stays finite over L = 200). The solve still returns OK; a row whose states
    are not all finite reports a non-finite row maximum and is not converged; a
    finite row matches the oracle to 1e-4 relative."""
    B, L, D = 2, 200, 64
    say(f"stress gru overflow B={B} L={L} D={D}")
    u = torch.zeros(B, L, 3, D)
    u[:, :, 1, :] = 5.0
    u[:, :, 2, :] = 0.1
    a = torch.zeros(3, D)
    a[2] = 8.0
    want, upd = O.newton("gru", u, a, K=3)
    assert np.isfinite(want).all() and np.abs(want).max() > 1e38  # beyond fp32, not fp64
    r = binding.solve("gru", u.to(DEV), a.to(DEV), iters=3)  # raises on a non-zero status
    torch.cuda.synchronize()
    got = r["h"].cpu().double().numpy()
    mu = r["max_update"].cpu().double().numpy()
    conv = r["converged"].cpu().numpy()
    assert int(r["iters"].item()) == 3
    for b in range(B):
        if np.isfinite(got[b]).all():
            scale = np.maximum(1.0, np.abs(want[0, b]))
            assert np.all(np.abs(got[b] - want[0, b]) <= 1e-4 * scale)
        else:
            assert not np.isfinite(mu[:, b]).all(), f"row {b}: non-finite states but finite row maxima"
            assert conv[b] == 0
    assert not np.isfinite(got).all(), "expected the fp32 iterate to overflow on this input"


@pytest.mark.parametrize("B,L,D", [(2, 200, 64), (2, 4096, 1024)])
def test_gru_zero_update_with_growing_jacobians(B, L, D):
    """u_c = 0 instead: the zero state is a fixed point of the cell, so the
    residual at the zero iterate is exactly 0 and so is every Newton update,
    while the Jacobians stay near 4.5. The scan composes products of Jacobians
    over a wave's steps (32 in the GRU's small-problem shape, 64 in the
    regular one); 4.5^64 passes the fp32 range, and such an infinite product
    applied to the zero carry gives inf * 0 = NaN. Either way no row may come
    back finite and wrong: a row is exactly 0 and converged, or it is
    non-finite, with a non-finite row maximum, and not converged."""
    say(f"stress gru zero update B={B} L={L} D={D} (plan {binding.plan('gru', binding.OP_SOLVE, B, L, D)})")
    u = torch.zeros(B, L, 3, D)
    u[:, :, 1, :] = 5.0
    a = torch.zeros(3, D)
    a[2] = 8.0
    r = binding.solve("gru", u.to(DEV), a.to(DEV), iters=3)
    torch.cuda.synchronize()
    got = r["h"].cpu().double().numpy()
    mu = r["max_update"].cpu().double().numpy()
    conv = r["converged"].cpu().numpy()
    for b in range(B):
        if np.isfinite(got[b]).all():
            assert np.all(got[b] == 0.0) and np.all(mu[:, b] == 0.0) and conv[b] == 1, f"row {b}"
        else:
            assert not np.isfinite(mu[:, b]).all() and conv[b] == 0, f"row {b}"
