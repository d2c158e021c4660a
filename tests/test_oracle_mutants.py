"""Plausible mistakes planted in copies of the oracle's C source must each fail at least one pin.

This shows the pins are sharp enough to catch a dropped term, a wrong sign, a wrong index or a
transposed operand. The mutants are compiled on the CPU into a temporary folder; the real oracle
is untouched. The multi-layer backward, composed in Python, gets the same treatment: mutated
copies of its source replace the method in a subclass of the oracle."""
import inspect
import os
import subprocess
import textwrap

import pytest

import oracle
from oracle_pins import ALL_PINS

SRC = open(oracle.SOURCE).read()

MUTANTS = {
    "sigmoid_sign": ("return 1.0 / (1.0 + exp(-x));", "return 1.0 / (1.0 + exp(x));"),
    "swap_i_f": ("const double ig = sigmoid(pre[0 * D + e]);", "const double ig = sigmoid(pre[1 * D + e]);"),
    "z_sigmoid": ("const double zg = tanh(pre[2 * D + e]);", "const double zg = sigmoid(pre[2 * D + e]);"),
    "R_transposed": ("for (long e = 0; e < D; ++e) a[e] += hd * row[e];",
                     "for (long e = 0; e < D; ++e) a[e] += hd * R[((g * N + n) * D + e) * D + d];"),
    "drop_bias": (" + a[e] + b[(g * N + n) * D + e];", " + a[e];"),
    "drop_Wx": ("Wx[(((bi * T + t) * G + g) * N + n) * D + e] + a[e]",
                "0.0 * Wx[(((bi * T + t) * G + g) * N + n) * D + e] + a[e]"),
    "wx_head0": ("Wx[(((bi * T + t) * G + g) * N + n) * D + e]", "Wx[(((bi * T + t) * G + g) * N + 0) * D + e]"),
    "c_uses_o": ("c[e] = fg * c[e] + ig * zg;", "c[e] = fg * c[e] + ig * og;"),
    "h_no_tanh": ("hn[e] = og * tanh(c[e]);", "hn[e] = og * c[e];"),
    "c0_ignored": ("c[e] = (S == 2 && states0) ? states0[((1 * B + bi) * N + n) * D + e] : 0.0;", "c[e] = 0.0;"),
    "h0_ignored": ("h[e] = states0 ? states0[((0 * B + bi) * N + n) * D + e] : 0.0;", "h[e] = 0.0;"),
    "states_time_reversed": ("states[(((0 * B + bi) * T + t) * N + n) * D + e] = h[e];",
                             "states[(((0 * B + bi) * T + (T - 1 - t)) * N + n) * D + e] = h[e];"),
    "elman_identity": ("for (long e = 0; e < D; ++e) hn[e] = tanh(pre[e]);",
                       "for (long e = 0; e < D; ++e) hn[e] = pre[e] / (1.0 + fabs(pre[e]));"),
    "async_update": ("memcpy(h, hn, sizeof(double) * D);", "memcpy(h, hn, sizeof(double) * D); h[0] = c[0];"),
    "gru_reset_dropped": ("tanh(Wx[(((bi * T + t) * G + 2) * N + n) * D + e] + rg * pre[2 * D + e])",
                          "tanh(Wx[(((bi * T + t) * G + 2) * N + n) * D + e] + pre[2 * D + e])"),
    "gru_reset_covers_wx": ("if (cell == ORACLE_CELL_GRU && g == 2) pre[g * D + e] = a[e] + b[(g * N + n) * D + e];",
                            "if (0) pre[g * D + e] = 0.0;"),
    "gru_bias_n_outside_reset": ("+ rg * pre[2 * D + e])",
                                 "+ rg * pre[2 * D + e] + (1.0 - rg) * b[(2 * N + n) * D + e])"),
    "gru_update_swapped": ("hn[e] = (1.0 - zg) * ng + zg * h[e];", "hn[e] = zg * ng + (1.0 - zg) * h[e];"),
    "gru_r_z_swapped": ("const double rg = sigmoid(pre[0 * D + e]);", "const double rg = sigmoid(pre[1 * D + e]);"),
    "gru_n_sigmoid": ("const double ng = tanh(Wx[", "const double ng = sigmoid(Wx["),
    "bwd_dc_carry_without_f": ("dc[e] = dct * fg;", "dc[e] = dct;"),
    "bwd_f_uses_c_t": ("dw[1] = dct * C[t * D + e] * fg * (1.0 - fg);", "dw[1] = dct * C[(t + 1) * D + e] * fg * (1.0 - fg);"),
    "bwd_tanh_derivative": ("dw[2] = dct * ig * (1.0 - zg * zg);", "dw[2] = dct * ig * (1.0 - zg);"),
    "bwd_o_uses_c_prev": ("const double tc = tanh(C[(t + 1) * D + e]);", "const double tc = tanh(C[t * D + e]);"),
    "bwd_dR_uses_h_after": ("const double hd = H[t * D + d];", "const double hd = H[(t + 1) * D + d];"),
    "bwd_R_transposed": ("for (long e = 0; e < D; ++e) s += dat[g * D + e] * row[e];",
                         "for (long e = 0; e < D; ++e) s += dat[g * D + e] * R[((g * N + n) * D + e) * D + d];"),
    "bwd_gru_da_n_without_r": ("dat[2 * D + e] = dq * rg;", "dat[2 * D + e] = dq;"),
    "bwd_gru_direct_dropped": ("dh[e] = dh[e] * zg;", "dh[e] = 0.0;"),
    "bwd_gru_dz_sign": ("const double dz = dh[e] * (H[t * D + e] - ng);", "const double dz = dh[e] * (ng - H[t * D + e]);"),
    "bwd_dlast_c_dropped": ("dc[e] = (S == 2 && dlast) ? dlast[((1 * B + bi) * N + n) * D + e] : 0.0;", "dc[e] = 0.0;"),
    "bwd_dstates_c_dropped": ("if (S == 2) dc[e] += dstates[(((1 * B + bi) * T + t) * N + n) * D + e];", ";"),
    "bwd_elman_derivative": ("dw[0] = dh[e] * (1.0 - ht * ht);", "dw[0] = dh[e] * (1.0 - ht);"),
    "bwd_db_skips_last_batch_row": ("for (long bi = 0; bi < B; ++bi) {\n            const long p = bi * N + n;\n            const double* DA",
                                    "for (long bi = 0; bi < B - 1; ++bi) {\n            const long p = bi * N + n;\n            const double* DA"),
    "stack_bias_hh_dropped": ("bias[l * H4 + j] = b_ih[l][j] + b_hh[l][j];", "bias[l * H4 + j] = b_ih[l][j];"),
    "stack_layer_input": ("const double* in = (l == 0) ? x + (t * B + bi) * I : h + (l - 1) * H;",
                          "const double* in = (l == 0) ? x + (t * B + bi) * I : h + l * H;"),
    "stack_wh_layer0": ("const double* row = Wh[l] + k * H4;", "const double* row = Wh[0] + k * H4;"),
    "stack_gate_blocks": ("const double gg = tanh(ifgo[2 * H + e]);", "const double gg = tanh(ifgo[3 * H + e]);"),
    "dirs_reverse_not_reversed": ("const long t = (k == 0) ? s : T - 1 - s;", "const long t = s;"),
    "dirs_concat_swapped": ("cur[t * W + k * H + e] = h[e];", "cur[t * W + (dirs - 1 - k) * H + e] = h[e];"),
    "dirs_reverse_uses_forward_weights": ("const long j = l * dirs + k;", "const long j = l * dirs;"),
    "dirs_next_layer_sees_direction0_only": ("const long K = (l == 0) ? I : W;", "const long K = (l == 0) ? I : H;"),
    "dirs_hn_direction_major": ("if (hn) hn[(j * B + bi) * H + e] = h[e];", "if (hn) hn[((k * L + l) * B + bi) * H + e] = h[e];"),
    "dirs_bias_hh_dropped": ("for (long q = 0; q < H4; ++q) ifgo[q] = b_ih[j][q] + b_hh[j][q];",
                             "for (long q = 0; q < H4; ++q) ifgo[q] = b_ih[j][q];"),
    "dirs_c_not_carried": ("c[e] = fg * c[e] + ig * gg;\n            h[e] = og * tanh(c[e]);\n            cur",
                           "c[e] = ig * gg;\n            h[e] = og * tanh(c[e]);\n            cur"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    assert SRC.count(old) >= 1, f"mutation anchor for {name} not found in the oracle source"
    src = tmp_path / f"oracle_{name}.c"
    src.write_text(SRC.replace(old, new))
    lib = str(tmp_path / f"liboracle_{name}.so")
    oracle.build(source=str(src), out=lib)
    mutant = oracle.Oracle(lib)
    caught_by = None
    for pin in ALL_PINS:
        try:
            pin(mutant)
        except (AssertionError, RuntimeError, ValueError):
            caught_by = pin.__name__
            break
    assert caught_by, f"mutant {name} passed every pin"


STACK_BWD_SRC = textwrap.dedent(inspect.getsource(oracle.Oracle.lstm_stack_bwd))

PY_MUTANTS = {
    "stack_bwd_reverse_dx_not_flipped": ("dXin += order(dproj @ Wi[j].T, k)", "dXin += dproj @ Wi[j].T"),
    "stack_bwd_reverse_input_not_flipped": ("Xk = order(X[l], k)", "Xk = X[l]"),
    "stack_bwd_dout_columns_swapped": ("order(dX[:, :, k * H:(k + 1) * H], k)",
                                       "order(dX[:, :, (dirs - 1 - k) * H:(dirs - k) * H], k)"),
    "stack_bwd_reverse_uses_forward_wi": ("dXin += order(dproj @ Wi[j].T, k)", "dXin += order(dproj @ Wi[l * dirs].T, k)"),
    "stack_bwd_dhn_direction_major": ("dlast[0, :, 0, 0] = _f64(dhn)[j]", "dlast[0, :, 0, 0] = _f64(dhn)[k * L + l]"),
    "stack_bwd_db_hh_zero": ("dbh[j] = dbi[j].copy()", "dbh[j] = 0.0 * dbi[j]"),
    "stack_bwd_dx_one_direction": ("dXin += order(", "dXin = order("),
    "stack_bwd_dcn_dropped": ("dlast[1, :, 0, 0] = _f64(dcn)[j]", "dlast[1, :, 0, 0] = 0.0"),
    "stack_bwd_forward_input_not_flipped": ("proj = order(X[l], k) @ Wi[j]", "proj = X[l] @ Wi[j]"),
}


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_stack_bwd_mutant_is_caught(name):
    old, new = PY_MUTANTS[name]
    assert STACK_BWD_SRC.count(old) >= 1, f"mutation anchor for {name} not found in lstm_stack_bwd"
    ns = dict(vars(oracle))
    exec(compile(STACK_BWD_SRC.replace(old, new), f"<mutant {name}>", "exec"), ns)
    mutant = type("MutantOracle", (oracle.Oracle,), {"lstm_stack_bwd": ns["lstm_stack_bwd"]})()
    caught_by = None
    for pin in ALL_PINS:
        try:
            pin(mutant)
        except (AssertionError, RuntimeError, ValueError):
            caught_by = pin.__name__
            break
    assert caught_by, f"mutant {name} passed every pin"
