"""The allocation-free ParaGRU solve (pararnn_solve_gru_scratch) against the
workspace entry point (pararnn_solve_gru), through the C ABI.

Two calls in a row on the library's built-in scratch, the second on a smaller
problem (the scratch keeps the first call's contents), each compared with the
workspace call on the same inputs and with the fp64 oracle: states within the
state tolerance, flags bit-exact under the margin rule."""
import numpy as np
import pytest
import torch

from nonlinear_rnn_solve_newton_amd import binding
from nonlinear_rnn_solve_newton_amd.workloads import make_inputs
from oracle import oracle as O
from tests.helpers import STATE_TOL, assert_close, check_flags, say

pytestmark = pytest.mark.gpu

# (B, L, D, with an initial state): the second call is smaller than the first
CALLS = [(4, 3000, 512, False), (1, 700, 96, True)]


@pytest.mark.parametrize("schedule", ["fused", "per_iteration"])
def test_scratch_solve_matches_workspace_solve(schedule):
    dev = torch.device("cuda:0")
    for i, (B, L, D, with_s0) in enumerate(CALLS):
        say(f"scratch solve, call {i + 1}: gru B={B} L={L} D={D} s0={with_s0} {schedule}")
        x = make_inputs("gru", B, L, D, seed=500 + 17 * i, u_dtype="bf16")
        u, a = x.u.to(dev), x.a.to(dev)
        s0 = np.random.default_rng(i).normal(size=(1, B, D)).astype(np.float32) if with_s0 else None
        h0 = torch.from_numpy(s0[0]).to(dev) if with_s0 else None
        ref = binding.solve("gru", u, a, h0=h0, iters=3, schedule=schedule)
        # outputs allocated up front: the scratch call itself allocates nothing
        h = torch.empty(B, L, D, dtype=torch.float32, device=dev)
        it = torch.empty(1, dtype=torch.int32, device=dev)
        conv = torch.empty(B, dtype=torch.int32, device=dev)
        mu = torch.empty(3, B, dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info(dev)[0]
        got = binding.solve_gru_scratch(u, a, h0=h0, iters=3, out=h, it=it, conv=conv, mu=mu,
                                        schedule=schedule)
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info(dev)[0] >= free0, "the scratch call took device memory"
        err = assert_close(got["h"].cpu().double().numpy(), ref["h"].cpu().double().numpy(), 1e-6,
                           "scratch vs workspace solve")
        assert int(got["iters"].item()) == int(ref["iters"].item()) == 3
        assert torch.equal(got["converged"], ref["converged"])
        assert_close(got["max_update"].cpu().double().numpy(), ref["max_update"].cpu().double().numpy(), 1e-6,
                     "max_update")
        want, upd = O.newton("gru", x.u, x.a, K=3, s0=None if s0 is None else s0.astype(np.float64))
        oerr = assert_close(got["h"].cpu().double().numpy()[None], want, STATE_TOL, "scratch solve vs oracle")
        check_flags(int(got["iters"].item()), got["converged"].cpu().numpy(), upd, 3, 1e-4)
        say(f"  vs workspace {err:.2e}, vs oracle {oerr:.2e}")


def test_scratch_solve_sizes_for_its_own_launch():
    """The long GRU workload (B=1 L=65536 D=2048) fits: its two-channel fused
    launch needs 38 MB of the 64 MiB scratch, though pararnn_workspace_bytes,
    which also covers the one-channel launch, asks for 152 MB. The result
    equals the workspace call's bit for bit (inclusive-only carries)."""
    dev = torch.device("cuda:0")
    B, L, D = 1, 65536, 2048
    assert binding.plan("gru", binding.OP_SOLVE, B, L, D)["inclusive_only"] == 1
    say(f"scratch solve: gru B={B} L={L} D={D} fused")
    x = make_inputs("gru", B, L, D, seed=77, u_dtype="bf16")
    u, a = x.u.to(dev), x.a.to(dev)
    ref = binding.solve("gru", u, a, iters=3, schedule="fused")
    got = binding.solve_gru_scratch(u, a, iters=3, schedule="fused")
    torch.cuda.synchronize()
    assert torch.equal(got["h"], ref["h"]) and torch.equal(got["converged"], ref["converged"])
    assert torch.equal(got["max_update"], ref["max_update"])


def test_scratch_solve_rejects_oversized_problem():
    """A problem whose workspace exceeds the scratch is refused before any launch."""
    dev = torch.device("cuda:0")
    u = torch.zeros(8, 4096, 3, 1024, dtype=torch.bfloat16, device=dev)
    a = torch.zeros(3, 1024, dtype=torch.float32, device=dev)
    with pytest.raises(binding.PararnnError, match="-5"):
        binding.solve_gru_scratch(u, a, schedule="per_iteration")
