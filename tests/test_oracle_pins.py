"""Pins of the fp64 oracle against facts fixed outside it (CPU only).

Each check ties the oracle to something other than itself:
  * hand-derived worked examples with exact gate values (tests/golden);
  * torch.nn.GRUCell / LSTMCell / GRU / LSTM in float64, which compute the same
    cells when their recurrent weights are diagonal and their input weights
    select the precomputed gate inputs;
  * central finite differences of the cell (Jacobian, input and coefficient
    derivatives);
  * brute-force dense Newton on tiny problems with numpy.linalg.solve, with the
    dense Jacobian taken by finite differences of the residual;
  * the linear-cell closed form (a = 0), where one Newton step is exact;
  * the fixed point of Newton equals the sequential trajectory, and after k
    iterations the first k rows are already exact (unit lower-bidiagonal
    Jacobian of the residual);
  * autograd through torch.nn.GRU / LSTM, finite differences of the loss, the
    dense adjoint solve, and the tangent/adjoint dot-product identity.
The method: ParaRNN article (cafecomtech.com), sections "O compromisso que SSMs
fizeram", "A sacada: método de Newton" and "Engenharia pra escalar".
"""
import json
import math
from pathlib import Path

import numpy as np
import pytest
import torch

from nonlinear_rnn_solve_newton_amd.workloads import make_inputs

GOLDEN = Path(__file__).resolve().parent / "golden" / "cell_worked_examples.json"
MATH_NS = {"log": math.log, "tanh": math.tanh, "exp": math.exp, "__builtins__": {}}


def ev(expr, **kw):
    return float(eval(expr, dict(MATH_NS), kw))  # closed forms from the golden file


# ---------------------------------------------------------------------------
# worked examples

def _golden():
    return json.loads(GOLDEN.read_text())


@pytest.mark.parametrize("case", _golden()["cells"], ids=lambda c: c["name"])
def test_cell_worked_example(oracle_lib, case):
    cell = case["cell"]
    s = np.array([[ev(x)] for x in case["s"]])
    u = np.array([[ev(x)] for x in case["u"]])
    a = np.array([[ev(x)] for x in case["a"]])
    out = oracle_lib.cell(cell, s, u, a)
    for key in ("f", "J", "dfdu", "dfda"):
        exp = np.array(case[key], dtype=object)
        got = out[key][..., 0]
        want = np.vectorize(ev, otypes=[float])(exp)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-14, err_msg=f"{case['name']} {key}")


@pytest.mark.parametrize("case", _golden()["sequences"], ids=lambda c: c["name"])
def test_sequence_worked_example(oracle_lib, case):
    cell, L = case["cell"], case["L"]
    G = len(case["u"])
    u = np.zeros((1, L, G, 1), np.float32)
    for g, x in enumerate(case["u"]):
        u[0, :, g, 0] = ev(x)
    a = np.array([[ev(x)] for x in case["a"]], np.float32)
    # the closed forms are evaluated on the float32-rounded inputs' exact gates:
    # recompute the gate constants from the rounded inputs to keep the pin exact
    uf = u[0, 0, :, 0].astype(np.float64)
    seq = oracle_lib.seq(cell, u, a)
    if cell == "gru":
        z = 1 / (1 + np.exp(-uf[0]))
        c = np.tanh(uf[2])
        want = np.array([[c * (1 - (1 - z) ** (l + 1)) for l in range(L)]])
        # same closed form written with the exact gate values, to 1e-7 (fp32 inputs)
        exact = np.array([[ev(case["states"][0][0], l=l) for l in range(L)]])
        np.testing.assert_allclose(want, exact, atol=1e-7)
        np.testing.assert_allclose(seq[:, 0, :, 0], want, atol=1e-14)
    else:
        i = 1 / (1 + np.exp(-uf[0]))
        f = 1 / (1 + np.exp(-uf[1]))
        o = 1 / (1 + np.exp(-uf[2]))
        g = np.tanh(uf[3])
        cs = np.array([i * g * (1 - f ** (l + 1)) / (1 - f) for l in range(L)])
        want = np.stack([cs, o * np.tanh(cs)])
        exact = np.array([[ev(case["states"][k][0], l=l) for l in range(L)] for k in range(2)])
        np.testing.assert_allclose(want, exact, atol=1e-7)
        np.testing.assert_allclose(seq[:, 0, :, 0], want, atol=1e-14)


# ---------------------------------------------------------------------------
# equivalence with torch.nn cells (float64)

def _torch_gru(a, D):
    """nn.GRU whose step equals the diagonal ParaGRU cell on inputs u = (u_z, u_r, u_c).

    torch: r = s(W_ir x + W_hr h), z_t = s(W_iz x + W_hz h), n = tanh(W_in x + r * (W_hn h)),
    h' = (1 - z_t) n + z_t h.  With z_t = 1 - z (so W_iz selects -u_z, W_hz = -diag(a_z)),
    n = c~ and W_hn = diag(a_c) this is h' = (1 - z) h + z c~.
    """
    gru = torch.nn.GRU(3 * D, D, batch_first=True, bias=False).double()
    I = torch.eye(D, dtype=torch.float64)
    Z = torch.zeros(D, D, dtype=torch.float64)
    a = torch.as_tensor(a, dtype=torch.float64)
    with torch.no_grad():
        gru.weight_ih_l0.copy_(torch.cat([torch.cat([Z, I, Z], 1),      # r <- u_r
                                          torch.cat([-I, Z, Z], 1),     # z_t <- -u_z
                                          torch.cat([Z, Z, I], 1)], 0))  # n <- u_c
        gru.weight_hh_l0.copy_(torch.cat([torch.diag(a[1]), torch.diag(-a[0]), torch.diag(a[2])], 0))
    return gru


def _torch_lstm(a, D):
    """nn.LSTM (gate order i, f, g, o) whose step equals the diagonal ParaLSTM cell."""
    lstm = torch.nn.LSTM(4 * D, D, batch_first=True, bias=False).double()
    I = torch.eye(D, dtype=torch.float64)
    Z = torch.zeros(D, D, dtype=torch.float64)
    a = torch.as_tensor(a, dtype=torch.float64)
    sel = lambda k: torch.cat([I if j == k else Z for j in range(4)], 1)  # noqa: E731
    with torch.no_grad():
        # our gate order (i, f, o, g) -> torch's (i, f, g, o)
        lstm.weight_ih_l0.copy_(torch.cat([sel(0), sel(1), sel(3), sel(2)], 0))
        lstm.weight_hh_l0.copy_(torch.cat([torch.diag(a[0]), torch.diag(a[1]),
                                           torch.diag(a[3]), torch.diag(a[2])], 0))
    return lstm


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_sequential_matches_torch_nn(oracle_lib, cell):
    B, L, D = 3, 40, 5
    x = make_inputs(cell, B, L, D, seed=11, u_dtype="f32", amax=1.5)
    G = x.u.shape[2]
    s0 = np.random.default_rng(3).normal(size=(2 if cell == "lstm" else 1, B, D))
    got = oracle_lib.seq(cell, x.u, x.a, s0=s0)
    inp = x.u.double().reshape(B, L, G * D)
    with torch.no_grad():
        if cell == "gru":
            y, _ = _torch_gru(x.a, D)(inp, torch.as_tensor(s0[0:1]))
            np.testing.assert_allclose(got[0], y.numpy(), atol=1e-13)
        else:
            y, _ = _torch_lstm(x.a, D)(inp, (torch.as_tensor(s0[1:2]), torch.as_tensor(s0[0:1])))
            np.testing.assert_allclose(got[1], y.numpy(), atol=1e-13)
            # c is checked step by step with LSTMCell
            cellm = torch.nn.LSTMCell(G * D, D, bias=False).double()
            ref = _torch_lstm(x.a, D)
            with torch.no_grad():
                cellm.weight_ih.copy_(ref.weight_ih_l0)
                cellm.weight_hh.copy_(ref.weight_hh_l0)
            h = torch.as_tensor(s0[1])
            c = torch.as_tensor(s0[0])
            for l in range(L):
                h, c = cellm(inp[:, l], (h, c))
                np.testing.assert_allclose(got[0][:, l], c.numpy(), atol=1e-13)


# ---------------------------------------------------------------------------
# finite differences of the cell

@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_cell_derivatives_finite_differences(oracle_lib, cell):
    rng = np.random.default_rng(5)
    NS, G, n = (1, 3, 200) if cell == "gru" else (2, 4, 200)
    s = rng.normal(size=(NS, n)) * 1.5
    u = rng.normal(size=(G, n)) * 1.5
    a = rng.uniform(-1.2, 1.2, size=(G, n))
    out = oracle_lib.cell(cell, s, u, a)
    eps = 1e-6

    def fd(which, k):
        args = {"s": s, "u": u, "a": a}
        p = {kk: vv.copy() for kk, vv in args.items()}
        m = {kk: vv.copy() for kk, vv in args.items()}
        p[which][k] += eps
        m[which][k] -= eps
        return (oracle_lib.cell(cell, **p)["f"] - oracle_lib.cell(cell, **m)["f"]) / (2 * eps)

    for q in range(NS):
        np.testing.assert_allclose(out["J"][:, q], fd("s", q), atol=2e-8, err_msg=f"J col {q}")
    for g in range(G):
        np.testing.assert_allclose(out["dfdu"][:, g], fd("u", g), atol=2e-8, err_msg=f"dfdu {g}")
        np.testing.assert_allclose(out["dfda"][:, g], fd("a", g), atol=2e-8, err_msg=f"dfda {g}")


# ---------------------------------------------------------------------------
# brute-force dense Newton

def _residual(oracle_lib, cell, S, u, a, s0):
    """F(S)_l = S_l - f(S_{l-1}, u_l) for one batch row; S [NS][L][D]."""
    NS, L, D = S.shape
    prev = np.concatenate([s0[:, None, :], S[:, :-1, :]], axis=1)  # [NS][L][D]
    n = L * D
    G = u.shape[1]
    f = oracle_lib.cell(cell, prev.reshape(NS, n),
                        u.transpose(1, 0, 2).reshape(G, n),
                        np.repeat(a[:, None, :], L, axis=1).reshape(G, n))["f"]
    return S - f.reshape(NS, L, D)


def _dense_jac(fun, x, eps=1e-6):
    x = x.ravel()
    cols = []
    for k in range(x.size):
        xp = x.copy()
        xm = x.copy()
        xp[k] += eps
        xm[k] -= eps
        cols.append((fun(xp) - fun(xm)).ravel() / (2 * eps))
    return np.stack(cols, axis=1)


@pytest.mark.parametrize("cell,L,D", [("gru", 1, 1), ("gru", 6, 3), ("gru", 8, 2),
                                      ("lstm", 1, 2), ("lstm", 5, 3), ("lstm", 8, 1)])
def test_dense_newton_bruteforce(oracle_lib, cell, L, D):
    K = 4
    x = make_inputs(cell, 1, L, D, seed=7 + L, u_dtype="f32", amax=1.2)
    u = x.u.numpy()[0].astype(np.float64)  # [L][G][D]
    a = x.a.numpy().astype(np.float64)
    NS = 2 if cell == "lstm" else 1
    s0 = np.random.default_rng(L).normal(size=(NS, 1, D)) * 0.5
    _, upd, its = oracle_lib.newton(cell, x.u, x.a, K=K, s0=s0, return_iterates=True)
    S = np.zeros((NS, L, D))
    for k in range(K):
        F = lambda v: _residual(oracle_lib, cell, v.reshape(NS, L, D), u, a, s0[:, 0])  # noqa: E731
        JF = _dense_jac(F, S)
        # structure: dF_l/dS_m = 0 unless m in {l, l-1} and the same channel d
        idx = np.array([(q, l, d) for q in range(NS) for l in range(L) for d in range(D)])
        same_d = idx[:, None, 2] == idx[None, :, 2]
        near_l = (idx[None, :, 1] == idx[:, None, 1]) | (idx[None, :, 1] == idx[:, None, 1] - 1)
        assert np.abs(JF[~(same_d & near_l)]).max(initial=0) < 1e-9
        # diagonal block dF_l/dS_l is the identity
        diag = (idx[:, None, 1] == idx[None, :, 1]) & same_d
        same_q = idx[:, None, 0] == idx[None, :, 0]
        np.testing.assert_allclose(JF[diag], same_q[diag].astype(float), atol=1e-9)
        Sn = S - np.linalg.solve(JF, F(S).ravel()).reshape(S.shape)
        np.testing.assert_allclose(its[k][:, 0], Sn, atol=1e-8, err_msg=f"iterate {k + 1}")
        np.testing.assert_allclose(upd[k, 0], np.abs(Sn - S).max(), atol=1e-8)
        S = Sn


# ---------------------------------------------------------------------------
# linear-cell closed forms (a = 0): one Newton step is exact

def test_gru_linear_cell_closed_form(oracle_lib):
    B, L, D = 2, 300, 7
    x = make_inputs("gru", B, L, D, seed=21, u_dtype="bf16", a_zero=True)
    uf = x.u.double().numpy()
    z = 1 / (1 + np.exp(-uf[:, :, 0]))
    c = np.tanh(uf[:, :, 2])
    # h_l = sum_{m <= l} prod_{j=m+1..l} (1 - z_j) z_m c_m, written as an explicit sum
    logk = np.log1p(-z)  # log(1 - z)
    cum = np.cumsum(logk, axis=1)
    want = np.zeros((B, L, D))
    for l in range(L):
        w = np.exp(cum[:, l:l + 1] - cum[:, :l + 1])  # prod_{j=m+1..l}(1 - z_j), m = 0..l
        want[:, l] = (w * z[:, :l + 1] * c[:, :l + 1]).sum(axis=1)
    out, upd = oracle_lib.newton("gru", x.u, x.a, K=3)
    np.testing.assert_allclose(out[0], want, atol=1e-12)
    # Newton from zero reaches it in one step; the second update is zero
    assert upd[1].max() < 1e-14 and upd[2].max() < 1e-14
    np.testing.assert_allclose(oracle_lib.newton("gru", x.u, x.a, K=1)[0][0], want, atol=1e-12)


def test_lstm_linear_cell_closed_form(oracle_lib):
    B, L, D = 2, 200, 5
    x = make_inputs("lstm", B, L, D, seed=22, u_dtype="bf16", a_zero=True)
    uf = x.u.double().numpy()
    sg = lambda v: 1 / (1 + np.exp(-v))  # noqa: E731
    i, f, o, g = sg(uf[:, :, 0]), sg(uf[:, :, 1]), sg(uf[:, :, 2]), np.tanh(uf[:, :, 3])
    logf = np.cumsum(np.log(f), axis=1)
    cs = np.zeros((B, L, D))
    for l in range(L):
        w = np.exp(logf[:, l:l + 1] - logf[:, :l + 1])
        cs[:, l] = (w * i[:, :l + 1] * g[:, :l + 1]).sum(axis=1)
    hs = o * np.tanh(cs)
    _, _, its = oracle_lib.newton("lstm", x.u, x.a, K=3, return_iterates=True)
    # c rows are affine in the previous state: exact after one step; h after two
    np.testing.assert_allclose(its[0][0], cs, atol=1e-12)
    np.testing.assert_allclose(its[1][0], cs, atol=1e-12)
    np.testing.assert_allclose(its[1][1], hs, atol=1e-12)
    np.testing.assert_allclose(its[2][1], hs, atol=1e-12)


# ---------------------------------------------------------------------------
# fixed point and finite termination

@pytest.mark.parametrize("cell,K,tol", [("gru", 9, 1e-12), ("lstm", 11, 1e-11)])
def test_newton_fixed_point_is_sequential(oracle_lib, cell, K, tol):
    x = make_inputs(cell, 2, 257, 6, seed=31, u_dtype="bf16")
    seq = oracle_lib.seq(cell, x.u, x.a)
    out, upd = oracle_lib.newton(cell, x.u, x.a, K=K)
    np.testing.assert_allclose(out, seq, atol=tol)
    assert upd[-1].max() < tol


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_newton_finite_termination(oracle_lib, cell):
    L = 12
    x = make_inputs(cell, 2, L, 4, seed=41, u_dtype="f32", amax=1.3)
    NS = 2 if cell == "lstm" else 1
    s0 = np.random.default_rng(2).normal(size=(NS, 2, 4))
    seq = oracle_lib.seq(cell, x.u, x.a, s0=s0)
    _, _, its = oracle_lib.newton(cell, x.u, x.a, K=L, s0=s0, return_iterates=True)
    for k in range(1, L + 1):
        # after k iterations rows 0..k-1 equal the sequential result
        np.testing.assert_allclose(its[k - 1][:, :, :k], seq[:, :, :k], atol=1e-13)
        if k <= 3:  # later rows are not exact yet (quadratic convergence hides it later)
            assert np.abs(its[k - 1][:, :, k:] - seq[:, :, k:]).max() > 1e-6
    # L <= K: the K-iterate is the sequential result
    np.testing.assert_allclose(its[-1], seq, atol=1e-13)


# ---------------------------------------------------------------------------
# adjoint / BPTT

@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_adjoint_matches_torch_autograd(oracle_lib, cell):
    B, L, D = 2, 30, 4
    x = make_inputs(cell, B, L, D, seed=51, u_dtype="f32", adjoint=True)
    G = x.u.shape[2]
    NS = 2 if cell == "lstm" else 1
    s0 = np.random.default_rng(9).normal(size=(NS, B, D)) * 0.5
    S = oracle_lib.seq(cell, x.u, x.a, s0=s0)
    du, ds0, da = oracle_lib.adjoint(cell, x.u, x.a, S, x.dh, s0=s0)

    inp = x.u.double().reshape(B, L, G * D).clone().requires_grad_(True)
    net = _torch_gru(x.a, D) if cell == "gru" else _torch_lstm(x.a, D)
    h0 = torch.as_tensor(s0[NS - 1:NS].copy()).requires_grad_(True)
    if cell == "gru":
        y, _ = net(inp, h0)
    else:
        c0 = torch.as_tensor(s0[0:1].copy()).requires_grad_(True)
        y, _ = net(inp, (h0, c0))
    loss = (y * x.dh.double()).sum()
    loss.backward()
    np.testing.assert_allclose(du.reshape(B, L, G * D), inp.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(ds0[NS - 1], h0.grad[0].numpy(), atol=1e-12)
    if cell == "lstm":
        np.testing.assert_allclose(ds0[0], c0.grad[0].numpy(), atol=1e-12)
    Whh = net.weight_hh_l0.grad
    if cell == "gru":  # rows (r, z_t, n), z_t uses -a_z
        got = np.stack([-torch.diagonal(Whh[D:2 * D]).numpy(), torch.diagonal(Whh[:D]).numpy(),
                        torch.diagonal(Whh[2 * D:]).numpy()])
    else:  # rows (i, f, g, o)
        got = np.stack([torch.diagonal(Whh[k * D:(k + 1) * D]).numpy() for k in (0, 1, 3, 2)])
    np.testing.assert_allclose(da, got, atol=1e-12)


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_adjoint_finite_differences_of_loss(oracle_lib, cell):
    B, L, D = 1, 25, 3
    x = make_inputs(cell, B, L, D, seed=61, u_dtype="f32", adjoint=True)
    u64 = x.u.double().numpy()
    NS = 2 if cell == "lstm" else 1
    loss = lambda uu: float((oracle_lib.seq(cell, uu, x.a)[NS - 1] * x.dh.double().numpy()).sum())  # noqa: E731
    S = oracle_lib.seq(cell, x.u, x.a)
    du, _, _ = oracle_lib.adjoint(cell, x.u, x.a, S, x.dh)
    rng = np.random.default_rng(0)
    # the oracle takes float32 u: perturb by float32-representable steps
    for _ in range(12):
        l, g, d = rng.integers(L), rng.integers(u64.shape[2]), rng.integers(D)
        eps = 2.0 ** -10
        up, um = u64.copy(), u64.copy()
        up[0, l, g, d] += eps
        um[0, l, g, d] -= eps
        fd = (loss(up.astype(np.float32)) - loss(um.astype(np.float32))) / (2 * eps)
        assert abs(fd - du[0, l, g, d]) < 5e-6 * max(1, abs(fd)), (l, g, d, fd, du[0, l, g, d])


@pytest.mark.parametrize("cell,L,D", [("gru", 7, 2), ("lstm", 6, 2)])
def test_adjoint_dense_solve_at_newton_iterate(oracle_lib, cell, L, D):
    """At a state that is not the fixed point (the 3-iterate), the adjoint is the
    solution of J_F(S)^T Lambda = G with J_F the residual's Jacobian, and
    du = -(dF/du)^T Lambda; both Jacobians by finite differences."""
    x = make_inputs(cell, 1, L, D, seed=71, u_dtype="f32", adjoint=True)
    NS = 2 if cell == "lstm" else 1
    u = x.u.numpy()[0].astype(np.float64)
    a = x.a.numpy().astype(np.float64)
    s0 = np.zeros((NS, D))
    S3, _ = oracle_lib.newton(cell, x.u, x.a, K=3)
    S = S3[:, 0]
    JF = _dense_jac(lambda v: _residual(oracle_lib, cell, v.reshape(S.shape), u, a, s0), S)
    Fu = _dense_jac(lambda v: _residual(oracle_lib, cell, S, v.reshape(u.shape), a, s0), u)
    Gv = np.zeros((NS, L, D))
    Gv[NS - 1] = x.dh.numpy()[0]
    Lam = np.linalg.solve(JF.T, Gv.ravel())
    du_dense = -(Fu.T @ Lam).reshape(u.shape)
    du, _, _ = oracle_lib.adjoint(cell, x.u, x.a, S3, x.dh)
    np.testing.assert_allclose(du[0], du_dense, atol=1e-8)


@pytest.mark.parametrize("cell", ["gru", "lstm"])
def test_adjoint_dot_product_identity(oracle_lib, cell):
    """<dh, dH> = <du, du_tangent> for the tangent recurrence
    dS_l = J_l dS_{l-1} + (df/du)_l du_l along a fixed trajectory."""
    B, L, D = 1, 40, 3
    x = make_inputs(cell, B, L, D, seed=81, u_dtype="f32", adjoint=True)
    NS = 2 if cell == "lstm" else 1
    G = x.u.shape[2]
    S, _ = oracle_lib.newton(cell, x.u, x.a, K=3)  # any trajectory works
    du, _, _ = oracle_lib.adjoint(cell, x.u, x.a, S, x.dh)
    rng = np.random.default_rng(1)
    tu = rng.normal(size=(L, G, D))
    u = x.u.numpy()[0].astype(np.float64)
    prev = np.concatenate([np.zeros((NS, 1, D)), S[:, 0, :-1]], axis=1)
    t = np.zeros((NS, D))
    lhs = 0.0
    for l in range(L):
        e = oracle_lib.cell(cell, prev[:, l], u[l], x.a.numpy().astype(np.float64))
        t = np.einsum("rqn,qn->rn", e["J"], t) + np.einsum("rgn,gn->rn", e["dfdu"], tu[l])
        lhs += float((x.dh.numpy()[0, l] * t[NS - 1]).sum())
    rhs = float((du[0] * tu).sum())
    assert abs(lhs - rhs) < 1e-12 * max(1.0, abs(lhs))


# ---------------------------------------------------------------------------
# flags

def test_flags_definitions(oracle_lib):
    upd = np.array([[1.0, 2.0], [1e-3, 5e-5], [5e-5, 9e-5], [1e-7, 1e-9]])
    assert oracle_lib.flags(upd, 1e-4)[0] == 4
    assert list(oracle_lib.flags(upd, 1e-4)[1]) == [1, 1]
    it, conv = oracle_lib.flags(upd, 1e-4, early_exit=True)
    assert it == 3 and list(conv) == [1, 1]
    it, conv = oracle_lib.flags(upd[:2], 1e-4, early_exit=True)
    assert it == 2 and list(conv) == [0, 1]
    nan = np.array([[np.nan, 0.0]])
    assert list(oracle_lib.flags(nan, 1e-4)[1]) == [0, 1]


def test_newton_nan_propagates_to_update(oracle_lib):
    x = make_inputs("gru", 2, 20, 3, seed=3, u_dtype="f32")
    u = x.u.clone()
    u[1, 7, 0, 2] = float("nan")
    out, upd = oracle_lib.newton("gru", u, x.a, K=3)
    assert np.isnan(upd[:, 1]).all() and np.isfinite(upd[:, 0]).all()
    assert np.isnan(out[0, 1, 7:, 2]).all() and np.isfinite(out[0, 0]).all()


# ---------------------------------------------------------------------------
# The linear recurrence alone (O4, the scan tier): s_l = A_l s_{l-1} + b_l.

def test_scan_unit_coefficient_is_cumulative_sum(oracle_lib):
    """A = 1: s_l = s0 + b_0 + ... + b_l (numpy.cumsum)."""
    rng = np.random.default_rng(40)
    B, L, D = 2, 37, 3
    b = rng.normal(size=(B, L, D))
    s0 = rng.normal(size=(1, B, D))
    s = oracle_lib.scan(np.ones((B, L, D)), b, s0)
    np.testing.assert_allclose(s, s0[0][:, None, :] + np.cumsum(b, axis=1), rtol=0, atol=1e-12)


def test_scan_zero_coefficient_returns_inputs(oracle_lib):
    rng = np.random.default_rng(41)
    b = rng.normal(size=(2, 9, 4))
    s = oracle_lib.scan(np.zeros_like(b), b, rng.normal(size=(1, 2, 4)))
    assert np.array_equal(s, b)


def test_scan_constant_coefficients_geometric_closed_form(oracle_lib):
    """A = alpha, b = beta: s_l = alpha^(l+1) s0 + beta (1 - alpha^(l+1)) / (1 - alpha)."""
    B, L, D = 1, 50, 3
    alpha = np.array([0.5, -0.8, 0.97])
    beta = np.array([1.0, -2.0, 0.25])
    s0 = np.array([[[0.3, 1.5, -4.0]]])
    s = oracle_lib.scan(np.broadcast_to(alpha, (B, L, D)), np.broadcast_to(beta, (B, L, D)), s0)
    p = alpha[None, :] ** (np.arange(1, L + 1)[:, None])  # [L][D]
    want = p * s0[0, 0] + beta * (1.0 - p) / (1.0 - alpha)
    np.testing.assert_allclose(s[0], want, rtol=1e-12, atol=1e-12)


def test_scan_block_rotation_closed_form(oracle_lib):
    """A_l = R(theta) (rotation, rows first), b = 0: s_l = R((l+1) theta) s0.
    A transposed block would rotate the other way."""
    L, theta = 23, 0.3
    R = np.array([[np.cos(theta), -np.sin(theta)], [np.sin(theta), np.cos(theta)]])
    A = np.broadcast_to(R[:, :, None, None, None], (2, 2, 1, L, 1))
    s = oracle_lib.scan(A, np.zeros((2, 1, L, 1)), np.array([[[1.0]], [[0.0]]]))
    ang = theta * np.arange(1, L + 1)
    np.testing.assert_allclose(s[0, 0, :, 0], np.cos(ang), atol=1e-12)
    np.testing.assert_allclose(s[1, 0, :, 0], np.sin(ang), atol=1e-12)


@pytest.mark.parametrize("ns", [1, 2])
def test_scan_dense_bidiagonal_solve(oracle_lib, ns):
    """The whole recurrence is one block lower-bidiagonal linear system
    (I - subdiag(A_1 .. A_{L-1})) s = b + e_0 A_0 s0, solved by numpy.linalg.solve."""
    rng = np.random.default_rng(42 + ns)
    L = 7
    A = rng.uniform(-1.2, 1.2, size=(ns, ns, L))
    b = rng.normal(size=(ns, L))
    s0 = rng.normal(size=ns)
    M = np.eye(L * ns)
    for l in range(1, L):
        M[l * ns:(l + 1) * ns, (l - 1) * ns:l * ns] = -A[:, :, l]
    rhs = b.T.reshape(-1).copy()
    rhs[:ns] += A[:, :, 0] @ s0
    want = np.linalg.solve(M, rhs).reshape(L, ns).T  # [ns][L]
    if ns == 1:
        s = oracle_lib.scan(A[0, 0][None, :, None], b[0][None, :, None], s0.reshape(1, 1, 1))
        got = s[:, :, 0]
    else:
        s = oracle_lib.scan(A[:, :, None, :, None], b[:, None, :, None], s0.reshape(2, 1, 1))
        got = s[:, 0, :, 0]
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-11)


def test_scan_block_with_zero_coupling_is_two_diagonal_scans(oracle_lib):
    rng = np.random.default_rng(44)
    B, L, D = 2, 15, 3
    a = rng.uniform(-0.9, 0.9, size=(2, B, L, D))
    b = rng.normal(size=(2, B, L, D))
    s0 = rng.normal(size=(2, B, D))
    A = np.zeros((2, 2, B, L, D))
    A[0, 0], A[1, 1] = a[0], a[1]
    s = oracle_lib.scan(A, b, s0)
    for r in range(2):
        np.testing.assert_allclose(s[r], oracle_lib.scan(a[r], b[r], s0[r:r + 1]), rtol=0, atol=1e-14)


def test_scan_is_linear_in_inputs_and_initial_state(oracle_lib):
    rng = np.random.default_rng(45)
    A = rng.uniform(-1, 1, size=(2, 2, 1, 30, 2))
    b1, b2 = rng.normal(size=(2, 2, 1, 30, 2))
    s1, s2 = rng.normal(size=(2, 2, 1, 2))
    lhs = oracle_lib.scan(A, b1 + 2.0 * b2, s1 - s2)
    rhs = oracle_lib.scan(A, b1, s1) + 2.0 * oracle_lib.scan(A, b2, None) - oracle_lib.scan(A, 0 * b1, s2)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# The dense recurrence (O5): s_l = A_l s_{l-1} + b_l with an n x n matrix.

def test_dense_recurrence_cyclic_shift_closed_form(oracle_lib):
    """A = cyclic shift (A[r][r-1 mod n] = 1), b = 0: s_l = s0 shifted by l+1
    positions towards higher indices. The transposed matrix shifts the other way."""
    n, L = 5, 12
    P = np.zeros((n, n))
    for r in range(n):
        P[r, (r - 1) % n] = 1.0
    A = np.broadcast_to(P, (1, L, n, n))
    s0 = np.arange(1.0, n + 1.0)[None]
    s = oracle_lib.scan_dense(A, np.zeros((1, L, n)), s0)
    for l in range(L):
        np.testing.assert_array_equal(s[0, l], np.roll(s0[0], l + 1))


def test_dense_recurrence_scaled_identity_geometric(oracle_lib):
    """A = alpha I, b = beta: each component is the scalar geometric closed form."""
    n, L, alpha = 4, 40, 0.9
    beta = np.array([1.0, -2.0, 0.5, 3.0])
    s0 = np.array([[0.2, -1.0, 4.0, 0.0]])
    A = np.broadcast_to(alpha * np.eye(n), (1, L, n, n))
    s = oracle_lib.scan_dense(A, np.broadcast_to(beta, (1, L, n)), s0)
    p = alpha ** np.arange(1, L + 1)[:, None]
    np.testing.assert_allclose(s[0], p * s0[0] + beta * (1 - p) / (1 - alpha), rtol=1e-12, atol=1e-12)


def test_dense_recurrence_bidiagonal_solve(oracle_lib):
    """The recurrence as one block lower-bidiagonal system, numpy.linalg.solve."""
    rng = np.random.default_rng(60)
    L, n = 6, 4
    A = rng.normal(size=(L, n, n))
    b = rng.normal(size=(L, n))
    s0 = rng.normal(size=n)
    M = np.eye(L * n)
    for l in range(1, L):
        M[l * n:(l + 1) * n, (l - 1) * n:l * n] = -A[l]
    rhs = b.reshape(-1).copy()
    rhs[:n] += A[0] @ s0
    want = np.linalg.solve(M, rhs).reshape(L, n)
    got = oracle_lib.scan_dense(A[None], b[None], s0[None])[0]
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-10)


def test_dense_recurrence_linear_in_inputs(oracle_lib):
    rng = np.random.default_rng(61)
    A = rng.normal(size=(2, 25, 3, 3)) * 0.5
    b1, b2 = rng.normal(size=(2, 2, 25, 3))
    s1, s2 = rng.normal(size=(2, 2, 3))
    lhs = oracle_lib.scan_dense(A, b1 - 3.0 * b2, s1 + s2)
    rhs = oracle_lib.scan_dense(A, b1, s1) - 3.0 * oracle_lib.scan_dense(A, b2) + oracle_lib.scan_dense(A, 0 * b1, s2)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-11, atol=1e-11)
