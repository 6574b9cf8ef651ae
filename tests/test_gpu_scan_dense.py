"""GPU parity of the dense recurrence (pararnn_scan_dense through the C ABI,
chunk transfers on the matrix cores) against the fp64 oracle's plain loop, on
the same seeded inputs: max-abs error within 1e-4."""
import numpy as np
import pytest
import torch

from nonlinear_rnn_solve_newton_amd import binding
from nonlinear_rnn_solve_newton_amd.workloads import (DENSE_WORKLOADS, dense_workload_inputs,
                                                      make_dense_scan_inputs)
from oracle import oracle as O
from tests.helpers import STATE_TOL, assert_close, say

pytestmark = pytest.mark.gpu

# n = 1, odd and padded sizes, the full 32; L below, at and past one segment
# (16 steps) and one chunk (128), many chunks; the chunk carries stage 16
# chunks at a time: exactly one block (2048 steps), one past it, and 33
# chunks (a last block of one); ragged tails
SHAPES = [
    (1, 1, 1), (2, 3, 5), (1, 7, 32), (1, 63, 32), (3, 64, 17), (1, 65, 32), (2, 1000, 32),
    (2, 777, 8), (1, 4097, 31), (4, 300, 16), (1, 129, 2), (1, 2048, 32), (2, 2049, 20),
]


@pytest.mark.parametrize("with_s0", [False, True], ids=["s0_zero", "s0_given"])
@pytest.mark.parametrize("B,L,n", SHAPES, ids=[f"{b}x{l}x{n}" for b, l, n in SHAPES])
def test_scan_dense_matches_oracle(B, L, n, with_s0):
    say(f"scan dense B={B} L={L} n={n} s0={with_s0}")
    x = make_dense_scan_inputs(B, L, n, seed=4000 + B + 3 * L + 7 * n)
    d = torch.device("cuda:0")
    s0 = x.s0.to(d) if with_s0 else None
    r = binding.scan_dense(x.A.to(d), x.b.to(d), s0)
    torch.cuda.synchronize()
    want = O.scan_dense(x.A, x.b, x.s0 if with_s0 else None)
    assert_close(r["s"].cpu().double().numpy(), want, STATE_TOL, f"dense scan n={n}")


def test_scan_dense_nan_propagates():
    B, L, n = 2, 300, 16
    x = make_dense_scan_inputs(B, L, n, seed=71)
    bb = x.b.clone()
    bb[1, 120, 3] = float("nan")
    d = torch.device("cuda:0")
    s = binding.scan_dense(x.A.to(d), bb.to(d))["s"].cpu().double().numpy()
    want = O.scan_dense(x.A, bb)
    assert np.array_equal(np.isnan(s), np.isnan(want))
    fin = ~np.isnan(want)
    assert np.abs(s[fin] - want[fin]).max() <= STATE_TOL


def test_scan_dense_rejects_large_state():
    d = torch.device("cuda:0")
    A = torch.zeros(1, 4, 33, 33, device=d)
    with pytest.raises(binding.PararnnError):
        binding.scan_dense(A, torch.zeros(1, 4, 33, device=d))


@pytest.mark.parametrize("name", list(DENSE_WORKLOADS))
def test_scan_dense_workload(name):
    """The full-size dense workload in the benchmark's launch configuration,
    every output against the oracle's loop (one fp64 pass per batch row)."""
    w = DENSE_WORKLOADS[name]
    say(f"dense workload {name}")
    x = dense_workload_inputs(w)
    d = torch.device("cuda:0")
    r = binding.scan_dense(x.A.to(d), x.b.to(d), x.s0.to(d))
    torch.cuda.synchronize()
    want = O.scan_dense(x.A, x.b, x.s0)  # the whole workload: one fp64 loop per row
    assert_close(r["s"].cpu().double().numpy(), want, STATE_TOL, f"{name}")
