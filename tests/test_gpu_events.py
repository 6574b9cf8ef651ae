"""The optional timing events of the C ABI: each call stamps them in order,
the kernel starts and ends by the dispatch itself, so every interval is
non-negative and a launch's interval lies inside the call's. The events leave
the results as they are: equal up to the run-to-run rounding of the chunk
carry (the look-back composes whichever predecessor values are published)."""
import ctypes

import pytest
import torch

from nonlinear_rnn_solve_newton_amd import binding
from nonlinear_rnn_solve_newton_amd.workloads import make_dense_scan_inputs, make_inputs, make_scan_inputs
from tests.helpers import say

RERUN_TOL = 1e-5  # two runs of one call: the carry's association may differ

pytestmark = pytest.mark.gpu


class Events:
    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
            self.ev.append(e.value)

    def ms(self, i, j):
        out = ctypes.c_float()
        assert self.hip.hipEventSynchronize(ctypes.c_void_p(self.ev[j])) == 0
        assert self.hip.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(self.ev[i]),
                                            ctypes.c_void_p(self.ev[j])) == 0
        return float(out.value)

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


def check_chain(ev, n):
    """Consecutive events are ordered and the whole span contains each step."""
    steps = [ev.ms(i, i + 1) for i in range(n - 1)]
    assert all(t >= 0.0 for t in steps), steps
    span = ev.ms(0, n - 1)
    assert span >= max(steps) - 1e-3, (span, steps)
    return steps


@pytest.mark.parametrize("schedule,early_exit", [("fused", False), ("per_iteration", False),
                                                 ("per_iteration", True)])
@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_solve_events(cell, schedule, early_exit):
    """Early exit runs a row-maximum kernel between the stamped launches."""
    say(f"events solve {cell} {schedule} early_exit={early_exit}")
    dev = torch.device("cuda:0")
    x = make_inputs(cell, 2, 4096, 256, seed=77, u_dtype="bf16")
    u, a = x.u.to(dev), x.a.to(dev)
    K = 3
    ev = Events(K + 2)
    try:
        r = binding.solve(cell, u, a, iters=K, schedule=schedule, early_exit=early_exit)
        ref = r["h"].clone()
        r2 = binding.solve(cell, u, a, iters=K, schedule=schedule, early_exit=early_exit, ws=r["ws"],
                           events=ev.ev)
        torch.cuda.synchronize()
        assert float((r2["h"] - ref).abs().max()) <= RERUN_TOL
        steps = check_chain(ev, K + 2)
        assert steps[1] > 0.0  # event 1 .. 2: the first (fused: the only) launch
        if schedule == "per_iteration":
            assert all(t > 0.0 for t in steps[1:]), steps
    finally:
        ev.close()


@pytest.mark.parametrize("want_da", [False, True])
def test_adjoint_events(want_da):
    say(f"events adjoint want_da={want_da}")
    dev = torch.device("cuda:0")
    x = make_inputs("gru", 2, 4096, 256, seed=78, u_dtype="bf16", adjoint=True)
    u, a, dh = x.u.to(dev), x.a.to(dev), x.dh.to(dev)
    h = binding.solve("gru", u, a, iters=3)["h"]
    ev = Events(3)
    try:
        ref = binding.adjoint("gru", u, a, h, dh, want_da=want_da)
        g = binding.adjoint("gru", u, a, h, dh, want_da=want_da, events=ev.ev)
        torch.cuda.synchronize()
        assert float((g["du"] - ref["du"]).abs().max()) <= RERUN_TOL
        if want_da:
            assert float((g["da"] - ref["da"]).abs().max()) <= RERUN_TOL * max(1.0, float(ref["da"].abs().max()))
        steps = check_chain(ev, 3)
        assert steps[1] > 0.0
    finally:
        ev.close()


@pytest.mark.parametrize("kind", ["diag", "block2", "dense"])
def test_scan_events(kind):
    say(f"events scan {kind}")
    dev = torch.device("cuda:0")
    ev = Events(3)
    try:
        if kind == "dense":
            x = make_dense_scan_inputs(2, 1024, 32, seed=79)
            A, b, s0 = x.A.to(dev), x.b.to(dev), x.s0.to(dev)
            ref = binding.scan_dense(A, b, s0)["s"].clone()
            s = binding.scan_dense(A, b, s0, events=ev.ev)["s"]
        else:
            x = make_scan_inputs(1 if kind == "diag" else 2, 2, 4096, 256, seed=80)
            A, b, s0 = x.A.to(dev), x.b.to(dev), x.s0.to(dev)
            ref = binding.scan(A, b, s0)["s"].clone()
            s = binding.scan(A, b, s0, events=ev.ev)["s"]
        torch.cuda.synchronize()
        assert float((s - ref).abs().max()) <= RERUN_TOL
        steps = check_chain(ev, 3)
        assert steps[1] > 0.0
    finally:
        ev.close()


def test_fused_launch_interval_inside_step():
    """The stamped interval of the fused launch is the kernel alone: shorter
    than the whole call bracketed by markers on the stream."""
    say("events fused interval inside the call")
    dev = torch.device("cuda:0")
    x = make_inputs("gru", 8, 4096, 1024, seed=81, u_dtype="bf16")
    u, a = x.u.to(dev), x.a.to(dev)
    ev = Events(5)
    try:
        r = binding.solve("gru", u, a, iters=3, schedule="fused")
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        best_launch, best_call = 1e9, 1e9
        for _ in range(5):
            torch.cuda.synchronize()
            start.record()
            binding.solve("gru", u, a, iters=3, schedule="fused", ws=r["ws"], out={"h": r["h"]}, events=ev.ev)
            stop.record()
            torch.cuda.synchronize()
            best_launch = min(best_launch, ev.ms(1, 2))
            best_call = min(best_call, start.elapsed_time(stop))
        assert 0.0 < best_launch < best_call, (best_launch, best_call)
    finally:
        ev.close()
