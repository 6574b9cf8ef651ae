"""GPU parity of the linear scan alone (pararnn_scan_diag / pararnn_scan_block2
through the C ABI) against the fp64 oracle's plain loop, on the same seeded
inputs: max-abs error within 1e-4 on the fp32 states."""
import numpy as np
import pytest
import torch

from nonlinear_rnn_solve_newton_amd import binding
from nonlinear_rnn_solve_newton_amd.workloads import (SCAN_WORKLOADS, make_scan_inputs,
                                                      scan_workload_inputs)
from oracle import oracle as O
from tests.helpers import STATE_TOL, assert_close, say

pytestmark = pytest.mark.gpu

# single step, tiny, odd D (one channel per lane), D % 4 == 2, ragged tiles and
# chunks, many chunks
SHAPES = [
    (1, 1, 1), (1, 2, 3), (2, 3, 2), (3, 5, 64), (1, 63, 65), (2, 64, 6), (1, 65, 4),
    (1, 127, 1000), (2, 128, 66), (1, 129, 128), (3, 1000, 64), (2, 1000, 200),
    (1, 4097, 3), (1, 5000, 130), (2, 300, 1000),
]


def _run(x, with_s0, **kw):
    d = torch.device("cuda:0")
    s0 = x.s0.to(d) if with_s0 else None
    r = binding.scan(x.A.to(d), x.b.to(d), s0, **kw)
    torch.cuda.synchronize()
    return r


@pytest.mark.parametrize("ns", [1, 2])
@pytest.mark.parametrize("with_s0", [False, True], ids=["s0_zero", "s0_given"])
@pytest.mark.parametrize("B,L,D", SHAPES, ids=[f"{b}x{l}x{d}" for b, l, d in SHAPES])
def test_scan_matches_oracle(ns, with_s0, B, L, D):
    say(f"scan ns={ns} s0={with_s0} B={B} L={L} D={D}")
    x = make_scan_inputs(ns, B, L, D, seed=2000 + 7 * B + 3 * L + D + ns)
    r = _run(x, with_s0)
    s0 = (x.s0 if ns == 2 else x.s0[None]) if with_s0 else None
    want = O.scan(x.A, x.b, s0)
    assert_close(r["s"].cpu().double().numpy(), want, STATE_TOL, f"scan ns={ns}")


@pytest.mark.parametrize("ns", [1, 2])
def test_scan_nan_propagates_along_its_channel(ns):
    say(f"scan ns={ns} NaN input")
    B, L, D = 2, 700, 96
    x = make_scan_inputs(ns, B, L, D, seed=51)
    bb = x.b.clone()
    if ns == 1:
        bb[1, 300, 7] = float("nan")
    else:
        bb[0, 1, 300, 7] = float("nan")
    d = torch.device("cuda:0")
    s = binding.scan(x.A.to(d), bb.to(d))["s"].cpu().double().numpy()
    want = O.scan(x.A, bb)
    assert np.array_equal(np.isnan(s), np.isnan(want))
    fin = ~np.isnan(want)
    assert np.abs(s[fin] - want[fin]).max() <= STATE_TOL


@pytest.mark.parametrize("ns", [1, 2])
def test_scan_repeat_and_workspace_reuse(ns):
    """Same inputs, same workspace: equal to rounding (the look-back's
    association may vary from run to run)."""
    x = make_scan_inputs(ns, 2, 3000, 256, seed=53)
    r1 = _run(x, True)
    s1 = r1["s"].clone()
    r2 = _run(x, True, ws=r1["ws"])
    assert float((s1 - r2["s"]).abs().max()) <= 1e-5


@pytest.mark.parametrize("ns", [1, 2])
def test_scan_misaligned_pointers_use_narrow_path(ns):
    """Planes at a 4-byte (not 16-byte) offset select the one-channel path."""
    B, L, D = 2, 300, 64
    x = make_scan_inputs(ns, B, L, D, seed=55)
    d = torch.device("cuda:0")
    n_a, n_b = x.A.numel(), x.b.numel()
    bufa = torch.empty(n_a + 1, dtype=torch.float32, device=d)
    bufb = torch.empty(n_b + 1, dtype=torch.float32, device=d)
    A = bufa[1:].view(x.A.shape)
    b = bufb[1:].view(x.b.shape)
    A.copy_(x.A.to(d))
    b.copy_(x.b.to(d))
    out = torch.empty(n_b + 1, dtype=torch.float32, device=d)[1:].view(x.b.shape)
    binding.scan(A, b, out=out)
    torch.cuda.synchronize()
    assert_close(out.cpu().double().numpy(), O.scan(x.A, x.b), STATE_TOL, "misaligned scan")


@pytest.mark.parametrize("name", list(SCAN_WORKLOADS))
def test_scan_workload_every_element(name):
    """Full-size scan workloads in the benchmark's launch configuration, every
    element against the oracle's loop (tile by tile over channels, all batch
    rows and the full L per tile)."""
    w = SCAN_WORKLOADS[name]
    say(f"scan workload {name}")
    x = scan_workload_inputs(w)
    r = _run(x, True)
    s = r["s"].cpu()
    err = 0.0
    DT = 256
    for d0 in range(0, w.D, DT):
        d1 = min(w.D, d0 + DT)
        if w.ns == 1:
            want = O.scan(x.A[..., d0:d1].contiguous(), x.b[..., d0:d1].contiguous(),
                          x.s0[None, :, d0:d1].contiguous())
        else:
            want = O.scan(x.A[..., d0:d1].contiguous(), x.b[..., d0:d1].contiguous(), x.s0[..., d0:d1].contiguous())
        err = max(err, assert_close(s[..., d0:d1].double().numpy(), want, STATE_TOL, f"{name} channels {d0}:{d1}"))
    say(f"scan workload {name}: every element within {err:.2e}")
