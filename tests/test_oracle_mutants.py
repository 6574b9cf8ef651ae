"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case rewrites one expression of pararnn_oracle.c into a plausible mistake
(a dropped term, a wrong sign, a wrong index, a transposed operand), builds the
modified copy in a temporary directory and runs the pins of
test_oracle_pins.py against it: at least one pin has to fail. The unmodified
source must contain each original expression, so the list stays in sync with
the code.
"""
import numpy as np
import pytest

from oracle import oracle as O
from tests import test_oracle_pins as P

MUTANTS = [
    ("gru_update_sign", "e->f[0] = (1.0 - z) * h + z * c;", "e->f[0] = (1.0 - z) * h - z * c;"),
    ("gru_reset_position", "double c = tanh(a[2] * (r * h) + u[2]);",
     "double c = tanh(a[2] * h + r * u[2]);"),
    ("gru_jacobian_dropped_reset_term", "g_c * a[2] * (r + h * dr * a[1]);", "g_c * a[2] * r;"),
    ("gru_dfda_c_missing_r", "e->dfda[0][2] = g_c * r * h;", "e->dfda[0][2] = g_c * h;"),
    ("lstm_gate_swap", "double g = tanh(a[3] * hp + u[3]);", "double g = tanh(a[2] * hp + u[2]);"),
    ("lstm_jhc_missing_f", "e->J[1][0] = q * f;", "e->J[1][0] = q;"),
    ("lstm_x_dropped_term", "double X = dci * a[0] + dcf * a[1] + dcg * a[3];",
     "double X = dci * a[0] + dcg * a[3];"),
    ("newton_offset_sign", "bv[(size_t)l * NS + r] = e.f[r] - jp;", "bv[(size_t)l * NS + r] = e.f[r] + jp;"),
    ("newton_linearise_wrong_row", "(l == 0) ? s0 : &S[(size_t)(l - 1) * NS];",
     "(l == 0) ? s0 : &S[(size_t)l * NS];"),
    ("newton_transposed_block", "acc += A[((size_t)l * NS + r) * NS + q] * prev[q];",
     "acc += A[((size_t)l * NS + q) * NS + r] * prev[q];"),
    ("newton_update_size_wrong", "m = nan_max(m, fabs(Sn[x] - S[x]));", "m = nan_max(m, fabs(Sn[x]));"),
    ("adjoint_not_transposed", "for (int r = 0; r < NS; ++r) acc += e.J[r][q] * lam[r];",
     "for (int r = 0; r < NS; ++r) acc += e.J[q][r] * lam[r];"),
    ("adjoint_gradient_row_shift", "lam[NS - 1] += (double)c->dh[((size_t)b * L + (l - 1)) * p->D + d];",
     "lam[NS - 1] += (double)c->dh[((size_t)b * L + l) * p->D + d];"),
    ("seq_initial_state_ignored", "for (int k = 0; k < p->NS; ++k) s[k] = p->s0 ?",
     "for (int k = 0; k < p->NS; ++k) s[k] = 0 ?"),
    ("scan_transposed_block", "acc += c->A[(size_t)(r * c->ns + q) * plane + at] * prev[q];",
     "acc += c->A[(size_t)(q * c->ns + r) * plane + at] * prev[q];"),
    ("scan_initial_state_ignored", "prev[r] = c->s0 ? c->s0[((size_t)r * c->B + b) * c->D + d] : 0.0;",
     "prev[r] = 0.0;"),
    ("scan_state_not_advanced", "          prev[r] = next[r];\n", "\n"),
    ("dense_transposed", "for (int q = 0; q < n; ++q) acc += Al[(size_t)r * n + q] * prev[q];",
     "for (int q = 0; q < n; ++q) acc += Al[(size_t)q * n + r] * prev[q];"),
    ("dense_initial_state_ignored", "for (int r = 0; r < n; ++r) prev[r] = c->s0 ? c->s0[(size_t)b * n + r] : 0.0;",
     "for (int r = 0; r < n; ++r) prev[r] = 0.0;"),
    ("dense_input_dropped_first_step", "double acc = c->b[step * n + r];",
     "double acc = l ? c->b[step * n + r] : 0.0;"),
]


def _pins():
    """(name, callable) for every pin, with small fixed parameters."""
    golden = P._golden()
    pins = []
    for c in golden["cells"]:
        pins.append((f"worked_{c['name']}", lambda c=c: P.test_cell_worked_example(O, c)))
    for c in golden["sequences"]:
        pins.append((f"seq_{c['name']}", lambda c=c: P.test_sequence_worked_example(O, c)))
    for cell in ("gru", "lstm"):
        pins += [
            (f"torch_nn_{cell}", lambda cell=cell: P.test_sequential_matches_torch_nn(O, cell)),
            (f"fd_{cell}", lambda cell=cell: P.test_cell_derivatives_finite_differences(O, cell)),
            (f"dense_{cell}", lambda cell=cell: P.test_dense_newton_bruteforce(O, cell, 5, 2)),
            (f"termination_{cell}", lambda cell=cell: P.test_newton_finite_termination(O, cell)),
            (f"autograd_{cell}", lambda cell=cell: P.test_adjoint_matches_torch_autograd(O, cell)),
            (f"dense_adjoint_{cell}",
             lambda cell=cell: P.test_adjoint_dense_solve_at_newton_iterate(O, cell, 5, 2)),
            (f"dot_{cell}", lambda cell=cell: P.test_adjoint_dot_product_identity(O, cell)),
        ]
    pins += [
        ("scan_cumsum", lambda: P.test_scan_unit_coefficient_is_cumulative_sum(O)),
        ("scan_geometric", lambda: P.test_scan_constant_coefficients_geometric_closed_form(O)),
        ("scan_rotation", lambda: P.test_scan_block_rotation_closed_form(O)),
        ("scan_dense_1", lambda: P.test_scan_dense_bidiagonal_solve(O, 1)),
        ("scan_dense_2", lambda: P.test_scan_dense_bidiagonal_solve(O, 2)),
        ("dense_shift", lambda: P.test_dense_recurrence_cyclic_shift_closed_form(O)),
        ("dense_geometric", lambda: P.test_dense_recurrence_scaled_identity_geometric(O)),
        ("dense_solve", lambda: P.test_dense_recurrence_bidiagonal_solve(O)),
    ]
    pins.append(("gru_closed_form", lambda: P.test_gru_linear_cell_closed_form(O)))
    pins.append(("lstm_closed_form", lambda: P.test_lstm_linear_cell_closed_form(O)))
    return pins


@pytest.mark.parametrize("name,orig,mut", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, orig, mut):
    src = O.SRC.read_text()
    assert src.count(orig) == 1, f"expression for {name} not found once in the oracle source"
    lib = O.build_variant(src.replace(orig, mut), tmp_path / f"mut_{name}.so")
    caught = []
    with O.using(lib):
        for pin_name, pin in _pins():
            try:
                with np.errstate(all="ignore"):
                    pin()
            except (AssertionError, ValueError, np.linalg.LinAlgError):
                caught.append(pin_name)
    assert caught, f"no pin rejects the planted mistake {name}"
