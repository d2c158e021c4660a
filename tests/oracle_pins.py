"""Pins of the fp64 oracle to facts that do not come from the oracle itself.

Every pin takes an ``oracle.Oracle`` and raises AssertionError when the oracle disagrees. The same
pins run against the real oracle (tests/test_oracle_pins.py) and against deliberately broken copies
of its C source and of its Python-composed multi-layer backward (tests/test_oracle_mutants.py),
which must each fail at least one pin.

Kinds of pin:
* golden fixtures (tests/golden/*.txt): closed forms and hand-stepped scalar recurrences evaluated
  with 50-digit decimals, independent of the oracle's code;
* closed forms evaluated here with numpy (R = 0 geometric gating; saturated forget gate; GRU with
  R = 0, a saturated update gate, a shut reset gate);
* library special cases: torch.nn.LSTM / torch.nn.RNN / torch.nn.GRU in float64 (the "5.3 LSTM"
  page builds its weights from exactly that module's state_dict names);
* invariants: heads independent (= one wide head with block-diagonal R), batch permutation,
  continuation through last_states, T = 0, state bounds, row subsets;
* two formulations: the page's time-major multi-layer loop against a layer-major composition of
  head-wise runs, and against the layer-by-layer formulation the bidirectional stack uses;
* the bidirectional reading (torch.nn.LSTM(bidirectional=True) in float64, a time-reversed
  one-direction run, layer composition);
* the backward: torch autograd through float64 torch layers (head-wise cells with identity input
  weights, the one- and two-direction multi-layer LSTM), central finite differences of the pinned
  forwards, linearity in the cotangent, T = 0.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from golden_io import load

ATOL_GOLD = 5e-15


def _sig(x):
    return 1.0 / (1.0 + np.exp(-x))


# ----------------------------------------------------------------------------- golden fixtures
def pin_golden_pre_0010(orc):
    """R = 0, pre = (0, 0, 1, 0): c_t = tanh(1)(1 - 2^-t), h_t = tanh(c_t)/2."""
    g = load("lstm_r0_pre_0010.txt")
    T = len(g["c"])
    Wx = np.zeros((1, T, 4, 1, 1))
    Wx[0, :, 2, 0, 0] = 1.0
    st, last = orc.headwise_fwd("lstm", Wx, np.zeros((4, 1, 1, 1)), np.zeros((4, 1, 1)))
    np.testing.assert_allclose(st[0, 0, :, 0, 0], g["h"], rtol=0, atol=ATOL_GOLD)
    np.testing.assert_allclose(st[1, 0, :, 0, 0], g["c"], rtol=0, atol=ATOL_GOLD)
    np.testing.assert_allclose(last[:, 0, 0, 0, 0], [g["h"][-1], g["c"][-1]], rtol=0, atol=ATOL_GOLD)


def pin_golden_general_const(orc):
    """R = 0, constant Wx and b split, nonzero c0 and h0: geometric closed form."""
    g = load("lstm_r0_general.txt")
    T = len(g["c"])
    Wx = np.zeros((1, T, 4, 1, 1))
    for k in range(4):
        Wx[0, :, k, 0, 0] = g["wx"][k]
    b = np.array(g["b"]).reshape(4, 1, 1)
    s0 = np.zeros((2, 1, 1, 1, 1))
    s0[0] = 0.3  # h0 is irrelevant when R = 0
    s0[1] = g["c0"][0]
    st, _ = orc.headwise_fwd("lstm", Wx, np.zeros((4, 1, 1, 1)), b, s0)
    np.testing.assert_allclose(st[1, 0, :, 0, 0], g["c"], rtol=0, atol=ATOL_GOLD)
    np.testing.assert_allclose(st[0, 0, :, 0, 0], g["h"], rtol=0, atol=ATOL_GOLD)


def pin_golden_elman_scalar(orc):
    """Elman D = 1: h_t = tanh(1 + 0.5 h_{t-1}), hand-stepped at 50 digits."""
    g = load("elman_scalar.txt")
    T = len(g["h"])
    Wx = np.ones((1, T, 1, 1, 1))
    R = np.full((1, 1, 1, 1), 0.5)
    st, last = orc.headwise_fwd("elman", Wx, R, np.zeros((1, 1, 1)))
    np.testing.assert_allclose(st[0, 0, :, 0, 0], g["h"], rtol=0, atol=ATOL_GOLD)
    assert last.shape == (1, 1, 1, 1, 1)


def pin_golden_gru_scalar(orc):
    """GRU D = 1 with nonzero recurrent weights, hand-stepped at 50 digits (gate order r, z, n)."""
    g = load("gru_scalar.txt")
    T = len(g["h"])
    Wx = np.zeros((1, T, 3, 1, 1))
    for k in range(3):
        Wx[0, :, k, 0, 0] = g["wx"][k]
    R = np.array(g["r"]).reshape(3, 1, 1, 1)
    b = np.array(g["b"]).reshape(3, 1, 1)
    s0 = np.array(g["h0"]).reshape(1, 1, 1, 1, 1)
    st, last = orc.headwise_fwd("gru", Wx, R, b, s0)
    np.testing.assert_allclose(st[0, 0, :, 0, 0], g["h"], rtol=0, atol=ATOL_GOLD)
    assert last.shape == (1, 1, 1, 1, 1)


def _tiny():
    g = load("lstm_tiny_d2_t4.txt")
    Wh = np.array(g["wh"]).reshape(2, 8)
    bias = np.array(g["bias"])
    xw = np.array(g["xw"]).reshape(4, 8)
    h = np.array(g["h"]).reshape(4, 2)
    c = np.array(g["c"]).reshape(4, 2)
    return g, Wh, bias, xw, h, c


def pin_golden_tiny_headwise(orc):
    """D = 2, T = 4 hand-stepped dense-form LSTM, mapped onto the head-wise layouts."""
    g, Wh, bias, xw, h, c = _tiny()
    Wx = np.zeros((1, 4, 4, 1, 2))
    R = np.zeros((4, 1, 2, 2))
    b = np.zeros((4, 1, 2))
    for gate in range(4):
        Wx[0, :, gate, 0, :] = xw[:, gate * 2:(gate + 1) * 2]
        R[gate, 0] = Wh[:, gate * 2:(gate + 1) * 2]
        b[gate, 0] = bias[gate * 2:(gate + 1) * 2]
    s0 = np.zeros((2, 1, 1, 1, 2))
    s0[0, 0, 0, 0] = g["h0"]
    s0[1, 0, 0, 0] = g["c0"]
    st, _ = orc.headwise_fwd("lstm", Wx, R, b, s0)
    np.testing.assert_allclose(st[0, 0, :, 0, :], h, rtol=0, atol=ATOL_GOLD)
    np.testing.assert_allclose(st[1, 0, :, 0, :], c, rtol=0, atol=ATOL_GOLD)


def pin_golden_tiny_stack(orc):
    """The same hand-stepped case through the page's dense multi-layer loop (Wi = identity)."""
    g, Wh, bias, xw, h, c = _tiny()
    x = xw.reshape(4, 1, 8)
    out, hn, cn = orc.lstm_stack_p3(x, [np.eye(8)], [Wh], [bias], [np.zeros(8)],
                                    np.array(g["h0"]).reshape(1, 1, 2), np.array(g["c0"]).reshape(1, 1, 2))
    np.testing.assert_allclose(out[:, 0, :], h, rtol=0, atol=ATOL_GOLD)
    np.testing.assert_allclose(cn[0, 0], c[-1], rtol=0, atol=ATOL_GOLD)
    np.testing.assert_allclose(hn[0, 0], h[-1], rtol=0, atol=ATOL_GOLD)


# ----------------------------------------------------------------------------- closed forms
def pin_closed_form_random_const(orc):
    """R = 0 and Wx constant over t: per unit c_t = f^t c0 + i z (1 - f^t)/(1 - f)."""
    rng = np.random.default_rng(11)
    B, T, N, D = 2, 30, 2, 8
    wx = rng.normal(size=(B, 1, 4, N, D))
    Wx = np.repeat(wx, T, axis=1)
    b = rng.normal(size=(4, N, D)) * 0.5
    s0 = rng.normal(size=(2, B, 1, N, D))
    st, _ = orc.headwise_fwd("lstm", Wx, np.zeros((4, N, D, D)), b, s0)
    pre = wx[:, 0] + b[None]  # [B,4,N,D]
    i, f, z, o = _sig(pre[:, 0]), _sig(pre[:, 1]), np.tanh(pre[:, 2]), _sig(pre[:, 3])
    for t in range(1, T + 1):
        ft = f ** t
        ct = ft * s0[1, :, 0] + i * z * (1 - ft) / (1 - f)
        np.testing.assert_allclose(st[1, :, t - 1], ct, rtol=0, atol=1e-12)
        np.testing.assert_allclose(st[0, :, t - 1], o * np.tanh(ct), rtol=0, atol=1e-12)


def pin_saturated_forget(orc):
    """b_f = +40, b_i = -40 (f rounds to 1, i ~ 4e-18): c stays c0, and with R[o] = 0,
    h_t = sigmoid(Wx_o[t] + b_o) tanh(c0)."""
    rng = np.random.default_rng(12)
    B, T, N, D = 3, 25, 2, 6
    Wx = rng.normal(size=(B, T, 4, N, D))
    Wx[:, :, 0:2] = 0.0
    R = rng.normal(size=(4, N, D, D)) * (0.5 / math.sqrt(D))
    R[3] = 0.0
    b = rng.normal(size=(4, N, D)) * 0.3
    b[0] = -40.0
    b[1] = 40.0
    s0 = rng.normal(size=(2, B, 1, N, D))
    st, _ = orc.headwise_fwd("lstm", Wx, R, b, s0)
    c0 = s0[1, :, 0]
    for t in range(T):
        np.testing.assert_allclose(st[1, :, t], c0, rtol=0, atol=(t + 1) * 1e-16 + 1e-15)
        h_exp = _sig(Wx[:, t, 3] + b[3][None]) * np.tanh(c0)
        np.testing.assert_allclose(st[0, :, t], h_exp, rtol=0, atol=1e-14)


def pin_elman_r0(orc):
    """Elman with R = 0 is the elementwise map h_t = tanh(Wx_t + b)."""
    rng = np.random.default_rng(13)
    B, T, N, D = 2, 9, 3, 5
    Wx = rng.normal(size=(B, T, 1, N, D))
    b = rng.normal(size=(1, N, D))
    st, _ = orc.headwise_fwd("elman", Wx, np.zeros((1, N, D, D)), b)
    np.testing.assert_allclose(st[0], np.tanh(Wx[:, :, 0] + b[0][None, None]), rtol=0, atol=1e-15)


def pin_gru_r0_closed_form(orc):
    """GRU with R = 0 and Wx constant over t: r, z, n are constant per unit and the update is an
    affine contraction, h_t = n + z^t (h0 - n) with n = tanh(Wx_n + r b_n)."""
    rng = np.random.default_rng(14)
    B, T, N, D = 2, 30, 2, 6
    wx = rng.normal(size=(B, 1, 3, N, D))
    Wx = np.repeat(wx, T, axis=1)
    b = rng.normal(size=(3, N, D)) * 0.7
    s0 = rng.normal(size=(1, B, 1, N, D))
    st, last = orc.headwise_fwd("gru", Wx, np.zeros((3, N, D, D)), b, s0)
    r = _sig(wx[:, 0, 0] + b[0][None])
    z = _sig(wx[:, 0, 1] + b[1][None])
    n = np.tanh(wx[:, 0, 2] + r * b[2][None])
    h0 = s0[0, :, 0]
    for t in range(1, T + 1):
        np.testing.assert_allclose(st[0, :, t - 1], n + z ** t * (h0 - n), rtol=0, atol=1e-14)
    np.testing.assert_array_equal(last[0, :, 0], st[0, :, -1])


def pin_gru_update_saturated(orc):
    """GRU with b_z = +40 (z = 1 - 4e-18): the state is carried through unchanged, whatever the
    candidate."""
    rng = np.random.default_rng(15)
    B, T, N, D = 3, 20, 2, 5
    Wx = rng.normal(size=(B, T, 3, N, D))
    Wx[:, :, 1] = 0.0
    R = rng.normal(size=(3, N, D, D)) * (0.5 / math.sqrt(D))
    R[1] = 0.0
    b = rng.normal(size=(3, N, D)) * 0.3
    b[1] = 40.0
    s0 = rng.normal(size=(1, B, 1, N, D)) * 0.5
    st, _ = orc.headwise_fwd("gru", Wx, R, b, s0)
    for t in range(T):
        np.testing.assert_allclose(st[0, :, t], s0[0, :, 0], rtol=0, atol=(t + 1) * 1e-16 + 1e-15)


def pin_gru_reset_closed(orc):
    """GRU with the reset gate shut (b_r = -40, no input or recurrent drive to r): the candidate is
    tanh(Wx_n), so the candidate's recurrent weights and bias no longer matter, while z still does."""
    rng = np.random.default_rng(16)
    B, T, N, D = 2, 12, 2, 5
    Wx = rng.normal(size=(B, T, 3, N, D))
    Wx[:, :, 0] = 0.0
    R = rng.normal(size=(3, N, D, D)) / math.sqrt(D)
    R[0] = 0.0
    b = rng.normal(size=(3, N, D)) * 0.3
    b[0] = -40.0
    s0 = rng.normal(size=(1, B, 1, N, D)) * 0.5
    st, _ = orc.headwise_fwd("gru", Wx, R, b, s0)
    R2, b2 = R.copy(), b.copy()
    R2[2] = rng.normal(size=(N, D, D))
    b2[2] = rng.normal(size=(N, D))
    st2, _ = orc.headwise_fwd("gru", Wx, R2, b2, s0)
    np.testing.assert_allclose(st2, st, rtol=0, atol=1e-14)
    # stepped here: h' = (1 - z) tanh(Wx_n) + z h, z = sigmoid(Wx_z + h.R_z + b_z)
    h = s0[0, :, 0]
    for t in range(T):
        az = np.einsum("bnd,nde->bne", h, R[1])
        z = _sig(Wx[:, t, 1] + az + b[1][None])
        h = (1 - z) * np.tanh(Wx[:, t, 2]) + z * h
        np.testing.assert_allclose(st[0, :, t], h, rtol=0, atol=1e-13)


# ----------------------------------------------------------------------------- library cases
def _torch_lstm(I, H, layers, seed):
    torch.manual_seed(seed)
    m = torch.nn.LSTM(I, H, num_layers=layers, dtype=torch.float64)
    return m


def pin_torch_lstm_stack(orc):
    """The page's MyLSTM reads weight_ih_l{k}.T, weight_hh_l{k}.T, bias_ih + bias_hh from a
    torch.nn.LSTM state_dict; in float64 the two must agree."""
    T, B, I, H, L = 7, 3, 5, 4, 2
    m = _torch_lstm(I, H, L, 21)
    rng = np.random.default_rng(21)
    x = rng.normal(size=(T, B, I))
    h0 = rng.normal(size=(L, B, H))
    c0 = rng.normal(size=(L, B, H))
    with torch.no_grad():
        ref, (rh, rc) = m(torch.from_numpy(x), (torch.from_numpy(h0), torch.from_numpy(c0)))
    sd = m.state_dict()
    Wi = [sd[f"weight_ih_l{l}"].numpy().T for l in range(L)]
    Wh = [sd[f"weight_hh_l{l}"].numpy().T for l in range(L)]
    bi = [sd[f"bias_ih_l{l}"].numpy() for l in range(L)]
    bh = [sd[f"bias_hh_l{l}"].numpy() for l in range(L)]
    out, hn, cn = orc.lstm_stack_p3(x, Wi, Wh, bi, bh, h0, c0)
    np.testing.assert_allclose(out, ref.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(hn, rh.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(cn, rc.numpy(), rtol=0, atol=1e-12)


def pin_torch_lstm_headwise(orc):
    """N independent torch.nn.LSTM layers (one per head) equal one head-wise run with
    Wx[b,t,g,n,:] = (x_n W_ih^T)[b, gH:(g+1)H], R[g,n,d,e] = W_hh[gH+e, d], b = b_ih + b_hh."""
    T, B, I, H, N = 6, 3, 4, 5, 3
    rng = np.random.default_rng(22)
    Wx = np.zeros((B, T, 4, N, H))
    R = np.zeros((4, N, H, H))
    b = np.zeros((4, N, H))
    s0 = rng.normal(size=(2, B, 1, N, H))
    refs_h, refs_c = [], []
    for n in range(N):
        m = _torch_lstm(I, H, 1, 100 + n)
        sd = m.state_dict()
        x = rng.normal(size=(T, B, I))
        with torch.no_grad():
            ref, (rh, rc) = m(torch.from_numpy(x), (torch.from_numpy(s0[0, :, 0, n][None].copy()),
                                                   torch.from_numpy(s0[1, :, 0, n][None].copy())))
        proj = x @ sd["weight_ih_l0"].numpy().T  # [T,B,4H]
        whh = sd["weight_hh_l0"].numpy()
        bias = sd["bias_ih_l0"].numpy() + sd["bias_hh_l0"].numpy()
        for g in range(4):
            Wx[:, :, g, n, :] = proj[:, :, g * H:(g + 1) * H].transpose(1, 0, 2)
            R[g, n] = whh[g * H:(g + 1) * H, :].T
            b[g, n] = bias[g * H:(g + 1) * H]
        refs_h.append(ref.numpy())
        refs_c.append(rc.numpy()[0])
    st, last = orc.headwise_fwd("lstm", Wx, R, b, s0)
    for n in range(N):
        np.testing.assert_allclose(st[0, :, :, n].transpose(1, 0, 2), refs_h[n], rtol=0, atol=1e-12)
        np.testing.assert_allclose(last[1, :, 0, n], refs_c[n], rtol=0, atol=1e-12)


def pin_torch_rnn_elman(orc):
    """Elman heads equal torch.nn.RNN(nonlinearity='tanh') layers in float64."""
    T, B, I, H, N = 8, 2, 3, 4, 2
    rng = np.random.default_rng(23)
    Wx = np.zeros((B, T, 1, N, H))
    R = np.zeros((1, N, H, H))
    b = np.zeros((1, N, H))
    s0 = rng.normal(size=(1, B, 1, N, H))
    refs = []
    for n in range(N):
        torch.manual_seed(200 + n)
        m = torch.nn.RNN(I, H, nonlinearity="tanh", dtype=torch.float64)
        sd = m.state_dict()
        x = rng.normal(size=(T, B, I))
        with torch.no_grad():
            ref, _ = m(torch.from_numpy(x), torch.from_numpy(s0[0, :, 0, n][None].copy()))
        Wx[:, :, 0, n, :] = (x @ sd["weight_ih_l0"].numpy().T).transpose(1, 0, 2)
        R[0, n] = sd["weight_hh_l0"].numpy().T
        b[0, n] = sd["bias_ih_l0"].numpy() + sd["bias_hh_l0"].numpy()
        refs.append(ref.numpy())
    st, _ = orc.headwise_fwd("elman", Wx, R, b, s0)
    for n in range(N):
        np.testing.assert_allclose(st[0, :, :, n].transpose(1, 0, 2), refs[n], rtol=0, atol=1e-12)


def pin_torch_gru_headwise(orc):
    """GRU heads equal torch.nn.GRU layers in float64 (gates r, z, n; the reset gate multiplies
    W_hn h + b_hn), with Wx[b,t,g,n,:] = x W_ig^T + b_ig, R[g,n,d,e] = W_hg[e,d] and b = b_hg."""
    T, B, I, H, N = 7, 3, 4, 5, 3
    rng = np.random.default_rng(24)
    Wx = np.zeros((B, T, 3, N, H))
    R = np.zeros((3, N, H, H))
    b = np.zeros((3, N, H))
    s0 = rng.normal(size=(1, B, 1, N, H))
    refs, lasts = [], []
    for n in range(N):
        torch.manual_seed(300 + n)
        m = torch.nn.GRU(I, H, dtype=torch.float64)
        with torch.no_grad():  # biases of the default init are small; widen them so each one counts
            m.bias_ih_l0.mul_(4.0)
            m.bias_hh_l0.mul_(4.0)
        sd = m.state_dict()
        x = rng.normal(size=(T, B, I))
        with torch.no_grad():
            ref, rh = m(torch.from_numpy(x), torch.from_numpy(s0[0, :, 0, n][None].copy()))
        proj = x @ sd["weight_ih_l0"].numpy().T + sd["bias_ih_l0"].numpy()  # [T,B,3H]
        whh = sd["weight_hh_l0"].numpy()
        bhh = sd["bias_hh_l0"].numpy()
        for g in range(3):
            Wx[:, :, g, n, :] = proj[:, :, g * H:(g + 1) * H].transpose(1, 0, 2)
            R[g, n] = whh[g * H:(g + 1) * H, :].T
            b[g, n] = bhh[g * H:(g + 1) * H]
        refs.append(ref.numpy())
        lasts.append(rh.numpy()[0])
    st, last = orc.headwise_fwd("gru", Wx, R, b, s0)
    for n in range(N):
        np.testing.assert_allclose(st[0, :, :, n].transpose(1, 0, 2), refs[n], rtol=0, atol=1e-12)
        np.testing.assert_allclose(last[0, :, 0, n], lasts[n], rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- invariants
def _rand_problem(cell, B, T, N, D, seed, with_s0=True):
    rng = np.random.default_rng(seed)
    G, S = {"lstm": (4, 2), "elman": (1, 1), "gru": (3, 1)}[cell]
    Wx = rng.normal(size=(B, T, G, N, D))
    R = rng.normal(size=(G, N, D, D)) / math.sqrt(D)
    b = rng.normal(size=(G, N, D)) * 0.3
    s0 = rng.normal(size=(S, B, 1, N, D)) if with_s0 else None
    return Wx, R, b, s0


def pin_heads_blockdiag(orc):
    """N heads of width D == one head of width N*D whose R is block-diagonal."""
    for cell in ("lstm", "elman", "gru"):
        B, T, N, D = 2, 6, 3, 4
        Wx, R, b, s0 = _rand_problem(cell, B, T, N, D, 31)
        G = Wx.shape[2]
        Wx1 = Wx.reshape(B, T, G, 1, N * D)
        R1 = np.zeros((G, 1, N * D, N * D))
        for n in range(N):
            R1[:, 0, n * D:(n + 1) * D, n * D:(n + 1) * D] = R[:, n]
        st, last = orc.headwise_fwd(cell, Wx, R, b, s0)
        st1, last1 = orc.headwise_fwd(cell, Wx1, R1, b.reshape(G, 1, N * D),
                                      s0.reshape(s0.shape[0], B, 1, 1, N * D))
        np.testing.assert_allclose(st1.reshape(st.shape), st, rtol=0, atol=1e-14)
        np.testing.assert_allclose(last1.reshape(last.shape), last, rtol=0, atol=1e-14)


def pin_heads_separate(orc):
    """An N-head run equals N separate one-head runs."""
    B, T, N, D = 2, 5, 3, 4
    Wx, R, b, s0 = _rand_problem("lstm", B, T, N, D, 32)
    st, _ = orc.headwise_fwd("lstm", Wx, R, b, s0)
    for n in range(N):
        stn, _ = orc.headwise_fwd("lstm", Wx[:, :, :, n:n + 1], R[:, n:n + 1], b[:, n:n + 1],
                                  s0[:, :, :, n:n + 1])
        np.testing.assert_array_equal(stn[:, :, :, 0], st[:, :, :, n])


def pin_batch_permutation(orc):
    """Permuting batch rows permutes the outputs (rows never interact)."""
    B, T, N, D = 5, 6, 2, 4
    Wx, R, b, s0 = _rand_problem("lstm", B, T, N, D, 33)
    perm = np.array([3, 0, 4, 1, 2])
    st, last = orc.headwise_fwd("lstm", Wx, R, b, s0)
    stp, lastp = orc.headwise_fwd("lstm", Wx[perm], R, b, s0[:, perm])
    np.testing.assert_array_equal(stp, st[:, perm])
    np.testing.assert_array_equal(lastp, last[:, perm])


def pin_continuation(orc):
    """Feeding last_states back as the initial state continues the sequence exactly."""
    for cell in ("lstm", "elman", "gru"):
        B, T, N, D = 2, 16, 2, 4
        Wx, R, b, s0 = _rand_problem(cell, B, T, N, D, 34)
        st, last = orc.headwise_fwd(cell, Wx, R, b, s0)
        st1, last1 = orc.headwise_fwd(cell, Wx[:, :7], R, b, s0)
        st2, last2 = orc.headwise_fwd(cell, Wx[:, 7:], R, b, last1)
        np.testing.assert_array_equal(np.concatenate([st1, st2], axis=2), st)
        np.testing.assert_array_equal(last2, last)
        np.testing.assert_array_equal(last, st[:, :, -1:])


def pin_t0(orc):
    """T = 0: last_states is the initial state (zeros when none is given)."""
    B, N, D = 2, 2, 3
    Wx, R, b, s0 = _rand_problem("lstm", B, 0, N, D, 35)
    st, last = orc.headwise_fwd("lstm", Wx, R, b, s0)
    assert st.shape == (2, B, 0, N, D)
    np.testing.assert_array_equal(last, s0)
    _, last0 = orc.headwise_fwd("lstm", Wx, R, b, None)
    np.testing.assert_array_equal(last0, np.zeros_like(s0))


def pin_bounds(orc):
    """|h| <= 1 always; |c_t| <= |c0| + t (|i z| <= 1, 0 <= f <= 1)."""
    B, T, N, D = 3, 40, 2, 8
    Wx, R, b, s0 = _rand_problem("lstm", B, T, N, D, 36)
    Wx *= 5.0
    R *= 3.0
    st, _ = orc.headwise_fwd("lstm", Wx, R, b, s0)
    assert np.all(np.abs(st[0]) <= 1.0)
    for t in range(T):
        assert np.all(np.abs(st[1, :, t]) <= np.abs(s0[1, :, 0]) + (t + 1) + 1e-12)
    We, Re, be, se = _rand_problem("elman", B, T, N, D, 37)
    ste, _ = orc.headwise_fwd("elman", We * 5.0, Re * 3.0, be, se)
    assert np.all(np.abs(ste) <= 1.0)
    # GRU: h' is a convex combination of h and n in (-1, 1), so |h_t| <= max(1, |h0|), and the
    # step is a contraction towards (-1, 1): from |h0| > 1 the excess never grows
    Wg, Rg, bg, sg = _rand_problem("gru", B, T, N, D, 40)
    sg *= 3.0
    stg, _ = orc.headwise_fwd("gru", Wg * 5.0, Rg * 3.0, bg, sg)
    bound = np.maximum(1.0, np.abs(sg[0, :, 0]))
    prev = np.abs(sg[0, :, 0])
    for t in range(T):
        cur = np.abs(stg[0, :, t])
        assert np.all(cur <= bound + 1e-15)
        assert np.all(np.maximum(cur - 1.0, 0.0) <= np.maximum(prev - 1.0, 0.0) + 1e-15)
        prev = cur


def pin_pairs_subset(orc):
    """Computing a subset of (batch, head) rows gives exactly those rows of the full run."""
    B, T, N, D = 3, 5, 2, 4
    Wx, R, b, s0 = _rand_problem("lstm", B, T, N, D, 38)
    st, last = orc.headwise_fwd("lstm", Wx, R, b, s0)
    pairs = [5, 1, 2]
    sts, lasts = orc.headwise_fwd("lstm", Wx, R, b, s0, pairs=pairs)
    for p in pairs:
        bi, n = divmod(p, N)
        np.testing.assert_array_equal(sts[:, bi, :, n], st[:, bi, :, n])
        np.testing.assert_array_equal(lasts[:, bi, :, n], last[:, bi, :, n])


def pin_layer_major(orc):
    """The page's time-major multi-layer loop equals layer-major head-wise runs (projection of
    each layer's whole input sequence first, then its recurrence)."""
    T, B, I, H, L = 9, 3, 5, 4, 2
    rng = np.random.default_rng(39)
    x = rng.normal(size=(T, B, I))
    Wi = [rng.normal(size=(I, 4 * H)) * 0.4, rng.normal(size=(H, 4 * H)) * 0.4]
    Wh = [rng.normal(size=(H, 4 * H)) * 0.4 for _ in range(L)]
    bi = [rng.normal(size=4 * H) * 0.2 for _ in range(L)]
    bh = [rng.normal(size=4 * H) * 0.2 for _ in range(L)]
    h0 = rng.normal(size=(L, B, H))
    c0 = rng.normal(size=(L, B, H))
    out, hn, cn = orc.lstm_stack_p3(x, Wi, Wh, bi, bh, h0, c0)
    inp = x
    for l in range(L):
        proj = inp @ Wi[l]  # [T,B,4H]
        Wx = proj.reshape(T, B, 4, 1, H).transpose(1, 0, 2, 3, 4)
        R = Wh[l].reshape(H, 4, H).transpose(1, 0, 2)[:, None]  # R[g,0,d,e] = Wh[d, gH+e]
        b = (bi[l] + bh[l]).reshape(4, 1, H)
        s0 = np.stack([h0[l], c0[l]])[:, :, None, None, :]
        st, last = orc.headwise_fwd("lstm", Wx, R, b, s0)
        inp = st[0, :, :, 0].transpose(1, 0, 2)
        np.testing.assert_allclose(last[0, :, 0, 0], hn[l], rtol=0, atol=1e-12)
        np.testing.assert_allclose(last[1, :, 0, 0], cn[l], rtol=0, atol=1e-12)
    np.testing.assert_allclose(inp, out, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- bidirectional
def _torch_stack_weights(m, L, dirs):
    """The "5.3 LSTM" page's weight reading of a torch.nn.LSTM state_dict (weight_ih_l{k}.T,
    weight_hh_l{k}.T, bias_ih_l{k}, bias_hh_l{k}, and the "_reverse" ones of direction 1), in the
    oracle's order l * dirs + k."""
    sd = m.state_dict()
    sfx = ["", "_reverse"][:dirs]
    names = [(l, s) for l in range(L) for s in sfx]
    Wi = [sd[f"weight_ih_l{l}{s}"].numpy().T for l, s in names]
    Wh = [sd[f"weight_hh_l{l}{s}"].numpy().T for l, s in names]
    bi = [sd[f"bias_ih_l{l}{s}"].numpy() for l, s in names]
    bh = [sd[f"bias_hh_l{l}{s}"].numpy() for l, s in names]
    return Wi, Wh, bi, bh


def pin_torch_lstm_bidirectional(orc):
    """torch.nn.LSTM(bidirectional=True) in float64: two layers of two directions, initial
    states, outputs [T,B,2H] and final states [L*2,B,H] in its (layer, direction) order."""
    T, B, I, H, L = 7, 3, 5, 4, 2
    torch.manual_seed(23)
    m = torch.nn.LSTM(I, H, num_layers=L, bidirectional=True, dtype=torch.float64)
    rng = np.random.default_rng(23)
    x = rng.normal(size=(T, B, I))
    h0 = rng.normal(size=(2 * L, B, H))
    c0 = rng.normal(size=(2 * L, B, H))
    with torch.no_grad():
        ref, (rh, rc) = m(torch.from_numpy(x), (torch.from_numpy(h0), torch.from_numpy(c0)))
    Wi, Wh, bi, bh = _torch_stack_weights(m, L, 2)
    out, hn, cn = orc.lstm_stack_dirs(x, Wi, Wh, bi, bh, h0, c0, dirs=2)
    np.testing.assert_allclose(out, ref.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(hn, rh.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(cn, rc.numpy(), rtol=0, atol=1e-12)


def pin_stack_one_direction_is_the_page_loop(orc):
    """With one direction, the layer-by-layer formulation equals the page's time-major loop."""
    T, B, I, H, L = 8, 2, 6, 4, 3
    rng = np.random.default_rng(24)
    x = rng.normal(size=(T, B, I))
    Wi = [rng.normal(size=((I if l == 0 else H), 4 * H)) * 0.5 for l in range(L)]
    Wh = [rng.normal(size=(H, 4 * H)) * 0.5 for _ in range(L)]
    bi = [rng.normal(size=4 * H) * 0.3 for _ in range(L)]
    bh = [rng.normal(size=4 * H) * 0.3 for _ in range(L)]
    h0 = rng.normal(size=(L, B, H))
    c0 = rng.normal(size=(L, B, H))
    a = orc.lstm_stack_p3(x, Wi, Wh, bi, bh, h0, c0)
    b = orc.lstm_stack_dirs(x, Wi, Wh, bi, bh, h0, c0, dirs=1)
    for u, v in zip(a, b):
        np.testing.assert_allclose(v, u, rtol=0, atol=1e-13)


def pin_bidirectional_reverse_is_flipped_forward(orc):
    """Direction 1 of a layer equals a one-direction run over the time-reversed sequence with the
    reverse weights, reversed back; direction 0 equals a plain one-direction run."""
    T, B, I, H = 9, 3, 5, 4
    rng = np.random.default_rng(25)
    x = rng.normal(size=(T, B, I))
    Wi = [rng.normal(size=(I, 4 * H)) * 0.5 for _ in range(2)]
    Wh = [rng.normal(size=(H, 4 * H)) * 0.5 for _ in range(2)]
    bi = [rng.normal(size=4 * H) * 0.3 for _ in range(2)]
    bh = [rng.normal(size=4 * H) * 0.3 for _ in range(2)]
    h0 = rng.normal(size=(2, B, H))
    c0 = rng.normal(size=(2, B, H))
    out, hn, cn = orc.lstm_stack_dirs(x, Wi, Wh, bi, bh, h0, c0, dirs=2)
    f_out, f_hn, f_cn = orc.lstm_stack_p3(x, Wi[:1], Wh[:1], bi[:1], bh[:1], h0[:1], c0[:1])
    r_out, r_hn, r_cn = orc.lstm_stack_p3(x[::-1].copy(), Wi[1:], Wh[1:], bi[1:], bh[1:], h0[1:], c0[1:])
    np.testing.assert_allclose(out[:, :, :H], f_out, rtol=0, atol=1e-13)
    np.testing.assert_allclose(out[:, :, H:], r_out[::-1], rtol=0, atol=1e-13)
    np.testing.assert_allclose(hn, np.concatenate([f_hn, r_hn]), rtol=0, atol=1e-13)
    np.testing.assert_allclose(cn, np.concatenate([f_cn, r_cn]), rtol=0, atol=1e-13)


def pin_bidirectional_layers_compose(orc):
    """Two bidirectional layers equal one bidirectional layer fed the other's [T,B,2H] output."""
    T, B, I, H = 6, 2, 3, 4
    rng = np.random.default_rng(26)
    x = rng.normal(size=(T, B, I))
    Wi = [rng.normal(size=(I, 4 * H)) * 0.5 for _ in range(2)] + [rng.normal(size=(2 * H, 4 * H)) * 0.5 for _ in range(2)]
    Wh = [rng.normal(size=(H, 4 * H)) * 0.5 for _ in range(4)]
    bi = [rng.normal(size=4 * H) * 0.3 for _ in range(4)]
    bh = [rng.normal(size=4 * H) * 0.3 for _ in range(4)]
    out, hn, cn = orc.lstm_stack_dirs(x, Wi, Wh, bi, bh, dirs=2)
    o0, hn0, cn0 = orc.lstm_stack_dirs(x, Wi[:2], Wh[:2], bi[:2], bh[:2], dirs=2)
    o1, hn1, cn1 = orc.lstm_stack_dirs(o0, Wi[2:], Wh[2:], bi[2:], bh[2:], dirs=2)
    np.testing.assert_allclose(out, o1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(hn, np.concatenate([hn0, hn1]), rtol=0, atol=1e-13)
    np.testing.assert_allclose(cn, np.concatenate([cn0, cn1]), rtol=0, atol=1e-13)


# ----------------------------------------------------------------------------- backward
_GS = {"lstm": (4, 2), "elman": (1, 1), "gru": (3, 1)}


def _torch_identity_input_module(cell, H, seed):
    """A float64 torch recurrent layer whose input weight is the identity and input bias zero, so
    that its input x is exactly the head-wise Wx (torch's gate order: LSTM i, f, g, o; GRU r, z, n)
    and its recurrent-side weight and bias are R and b."""
    torch.manual_seed(seed)
    G = _GS[cell][0]
    if cell == "lstm":
        m = torch.nn.LSTM(G * H, H, dtype=torch.float64)
    elif cell == "gru":
        m = torch.nn.GRU(G * H, H, dtype=torch.float64)
    else:
        m = torch.nn.RNN(H, H, nonlinearity="tanh", dtype=torch.float64)
    with torch.no_grad():
        m.weight_ih_l0.copy_(torch.eye(G * H, dtype=torch.float64))
        m.bias_ih_l0.zero_()
        m.bias_hh_l0.mul_(4.0)
        m.weight_hh_l0.mul_(2.0)
    return m


def _pin_torch_autograd(orc, cell):
    """Backward of N heads equals torch autograd through N float64 torch layers, for the loss
    sum(dh * h_t) over all t + sum(dlast * last_states). torch returns c only at the end, so the
    per-step c gradient is zero here (finite differences cover it)."""
    G, S = _GS[cell]
    T, B, H, N = 6, 3, 4, 2
    rng = np.random.default_rng({"lstm": 51, "elman": 52, "gru": 53}[cell])
    Wx = rng.normal(size=(B, T, G, N, H))
    s0 = rng.normal(size=(S, B, 1, N, H)) * 0.7
    dstates = np.zeros((S, B, T, N, H))
    dstates[0] = rng.normal(size=(B, T, N, H))
    dlast = rng.normal(size=(S, B, 1, N, H))
    R = np.zeros((G, N, H, H))
    b = np.zeros((G, N, H))
    ref = {"dWx": np.zeros_like(Wx), "dR": np.zeros_like(R), "db": np.zeros_like(b), "ds0": np.zeros_like(s0)}
    for n in range(N):
        m = _torch_identity_input_module(cell, H, 400 + 10 * n + G)
        whh = m.weight_hh_l0.detach().numpy()
        bhh = m.bias_hh_l0.detach().numpy()
        for g in range(G):
            R[g, n] = whh[g * H:(g + 1) * H, :].T
            b[g, n] = bhh[g * H:(g + 1) * H]
        x = torch.tensor(Wx[:, :, :, n, :].reshape(B, T, G * H).transpose(1, 0, 2).copy(), requires_grad=True)
        h0 = torch.tensor(s0[0, :, 0, n][None].copy(), requires_grad=True)
        if cell == "lstm":
            c0 = torch.tensor(s0[1, :, 0, n][None].copy(), requires_grad=True)
            out, (hn, cn) = m(x, (h0, c0))
            loss = (out * torch.from_numpy(dstates[0, :, :, n].transpose(1, 0, 2).copy())).sum() \
                + (hn[0] * torch.from_numpy(dlast[0, :, 0, n].copy())).sum() \
                + (cn[0] * torch.from_numpy(dlast[1, :, 0, n].copy())).sum()
        else:
            out, hn = m(x, h0)
            loss = (out * torch.from_numpy(dstates[0, :, :, n].transpose(1, 0, 2).copy())).sum() \
                + (hn[0] * torch.from_numpy(dlast[0, :, 0, n].copy())).sum()
        loss.backward()
        gx = x.grad.numpy().transpose(1, 0, 2).reshape(B, T, G, H)
        ref["dWx"][:, :, :, n, :] = gx
        gw = m.weight_hh_l0.grad.numpy()
        gb = m.bias_hh_l0.grad.numpy()
        for g in range(G):
            ref["dR"][g, n] = gw[g * H:(g + 1) * H, :].T
            ref["db"][g, n] = gb[g * H:(g + 1) * H]
        ref["ds0"][0, :, 0, n] = h0.grad.numpy()[0]
        if cell == "lstm":
            ref["ds0"][1, :, 0, n] = c0.grad.numpy()[0]
    dWx, dR, db, ds0 = orc.headwise_bwd(cell, Wx, R, b, s0, dstates, dlast)
    np.testing.assert_allclose(dWx, ref["dWx"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dR, ref["dR"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(db, ref["db"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(ds0, ref["ds0"], rtol=0, atol=1e-12)


def pin_bwd_torch_lstm(orc):
    _pin_torch_autograd(orc, "lstm")


def pin_bwd_torch_gru(orc):
    _pin_torch_autograd(orc, "gru")


def pin_bwd_torch_elman(orc):
    _pin_torch_autograd(orc, "elman")


def _loss(orc, cell, Wx, R, b, s0, dstates, dlast):
    st, last = orc.headwise_fwd(cell, Wx, R, b, s0)
    return float((st * dstates).sum() + (last * dlast).sum())


def pin_bwd_finite_differences(orc):
    """Every gradient entry, on tiny problems of each cell with per-step c gradients, against
    central differences of the (independently pinned) forward: |error| <= 1e-7."""
    for cell, seed in (("lstm", 61), ("gru", 62), ("elman", 63)):
        G, S = _GS[cell]
        B, T, N, D = 2, 3, 2, 3
        rng = np.random.default_rng(seed)
        Wx = rng.normal(size=(B, T, G, N, D))
        R = rng.normal(size=(G, N, D, D)) * 0.6
        b = rng.normal(size=(G, N, D)) * 0.5
        s0 = rng.normal(size=(S, B, 1, N, D)) * 0.5
        dstates = rng.normal(size=(S, B, T, N, D))
        dlast = rng.normal(size=(S, B, 1, N, D))
        grads = orc.headwise_bwd(cell, Wx, R, b, s0, dstates, dlast)
        eps = 1e-5
        for k, arr in enumerate((Wx, R, b, s0)):
            num = np.zeros_like(arr)
            for idx in np.ndindex(arr.shape):
                old = arr[idx]
                arr[idx] = old + eps
                lp = _loss(orc, cell, Wx, R, b, s0, dstates, dlast)
                arr[idx] = old - eps
                lm = _loss(orc, cell, Wx, R, b, s0, dstates, dlast)
                arr[idx] = old
                num[idx] = (lp - lm) / (2 * eps)
            np.testing.assert_allclose(grads[k], num, rtol=0, atol=1e-7, err_msg=f"{cell} input {k}")


def pin_bwd_linear_in_cotangent(orc):
    """The backward is linear in (dstates, dlast), and zero cotangents give zero gradients."""
    for cell in ("lstm", "gru", "elman"):
        G, S = _GS[cell]
        B, T, N, D = 2, 5, 2, 4
        Wx, R, b, s0 = _rand_problem(cell, B, T, N, D, 64)
        rng = np.random.default_rng(65)
        d1, d2 = rng.normal(size=(S, B, T, N, D)), rng.normal(size=(S, B, T, N, D))
        l1, l2 = rng.normal(size=(S, B, 1, N, D)), rng.normal(size=(S, B, 1, N, D))
        g1 = orc.headwise_bwd(cell, Wx, R, b, s0, d1, l1)
        g2 = orc.headwise_bwd(cell, Wx, R, b, s0, d2, l2)
        g3 = orc.headwise_bwd(cell, Wx, R, b, s0, 2.0 * d1 - 3.0 * d2, 2.0 * l1 - 3.0 * l2)
        for a, c, e in zip(g1, g2, g3):
            np.testing.assert_allclose(e, 2.0 * a - 3.0 * c, rtol=1e-12, atol=1e-12)
        for z in orc.headwise_bwd(cell, Wx, R, b, s0, None, None):
            assert not np.any(z)


def pin_bwd_t0(orc):
    """T = 0: last_states is the initial state, so dstates0 = dlast and the rest is zero."""
    for cell in ("lstm", "gru"):
        G, S = _GS[cell]
        Wx, R, b, s0 = _rand_problem(cell, 2, 0, 2, 3, 66)
        dlast = np.random.default_rng(67).normal(size=(S, 2, 1, 2, 3))
        dWx, dR, db, ds0 = orc.headwise_bwd(cell, Wx, R, b, s0, None, dlast)
        assert dWx.shape == (2, 0, G, 2, 3) and not np.any(dR) and not np.any(db)
        np.testing.assert_array_equal(ds0, dlast)


def pin_bwd_torch_lstm_stack(orc):
    """The multi-layer backward equals torch autograd through a float64 two-layer torch.nn.LSTM
    (the module whose state_dict the "5.3 LSTM" page reads), for every gradient: x, Wi, Wh,
    both biases, h0 and c0."""
    T, B, I, H, L = 6, 3, 5, 4, 2
    m = _torch_lstm(I, H, L, 71)
    rng = np.random.default_rng(71)
    x = rng.normal(size=(T, B, I))
    h0 = rng.normal(size=(L, B, H)) * 0.5
    c0 = rng.normal(size=(L, B, H)) * 0.5
    dout = rng.normal(size=(T, B, H))
    dhn = rng.normal(size=(L, B, H))
    dcn = rng.normal(size=(L, B, H))
    xt = torch.tensor(x, requires_grad=True)
    h0t = torch.tensor(h0, requires_grad=True)
    c0t = torch.tensor(c0, requires_grad=True)
    out, (hn, cn) = m(xt, (h0t, c0t))
    loss = (out * torch.from_numpy(dout)).sum() + (hn * torch.from_numpy(dhn)).sum() + (cn * torch.from_numpy(dcn)).sum()
    loss.backward()
    sd = m.state_dict()
    Wi = [sd[f"weight_ih_l{l}"].numpy().T for l in range(L)]
    Wh = [sd[f"weight_hh_l{l}"].numpy().T for l in range(L)]
    bi = [sd[f"bias_ih_l{l}"].numpy() for l in range(L)]
    bh = [sd[f"bias_hh_l{l}"].numpy() for l in range(L)]
    dx, dWi, dWh, dbi, dbh, dh0, dc0 = orc.lstm_stack_bwd(x, Wi, Wh, bi, bh, h0, c0, dout, dhn, dcn)
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dh0, h0t.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dc0, c0t.grad.numpy(), rtol=0, atol=1e-12)
    for l in range(L):
        np.testing.assert_allclose(dWi[l], getattr(m, f"weight_ih_l{l}").grad.numpy().T, rtol=0, atol=1e-12)
        np.testing.assert_allclose(dWh[l], getattr(m, f"weight_hh_l{l}").grad.numpy().T, rtol=0, atol=1e-12)
        np.testing.assert_allclose(dbi[l], getattr(m, f"bias_ih_l{l}").grad.numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(dbh[l], getattr(m, f"bias_hh_l{l}").grad.numpy(), rtol=0, atol=1e-12)



def pin_bwd_torch_lstm_stack_bidirectional(orc):
    """The two-direction multi-layer backward equals torch autograd through a float64 two-layer
    torch.nn.LSTM(bidirectional=True) (reading A21), for every gradient: x, the Wi, Wh and both
    biases of each (layer, direction), h0 and c0 in its (layer, direction) order."""
    T, B, I, H, L = 6, 3, 5, 4, 2
    torch.manual_seed(73)
    m = torch.nn.LSTM(I, H, num_layers=L, bidirectional=True, dtype=torch.float64)
    rng = np.random.default_rng(73)
    x = rng.normal(size=(T, B, I))
    h0 = rng.normal(size=(2 * L, B, H)) * 0.5
    c0 = rng.normal(size=(2 * L, B, H)) * 0.5
    dout = rng.normal(size=(T, B, 2 * H))
    dhn = rng.normal(size=(2 * L, B, H))
    dcn = rng.normal(size=(2 * L, B, H))
    xt = torch.tensor(x, requires_grad=True)
    h0t = torch.tensor(h0, requires_grad=True)
    c0t = torch.tensor(c0, requires_grad=True)
    out, (hn, cn) = m(xt, (h0t, c0t))
    loss = (out * torch.from_numpy(dout)).sum() + (hn * torch.from_numpy(dhn)).sum() + (cn * torch.from_numpy(dcn)).sum()
    loss.backward()
    Wi, Wh, bi, bh = _torch_stack_weights(m, L, 2)
    dx, dWi, dWh, dbi, dbh, dh0, dc0 = orc.lstm_stack_bwd(x, Wi, Wh, bi, bh, h0, c0, dout, dhn, dcn, dirs=2)
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dh0, h0t.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dc0, c0t.grad.numpy(), rtol=0, atol=1e-12)
    names = [(l, s) for l in range(L) for s in ("", "_reverse")]
    for j, (l, s) in enumerate(names):
        np.testing.assert_allclose(dWi[j], getattr(m, f"weight_ih_l{l}{s}").grad.numpy().T, rtol=0, atol=1e-12)
        np.testing.assert_allclose(dWh[j], getattr(m, f"weight_hh_l{l}{s}").grad.numpy().T, rtol=0, atol=1e-12)
        np.testing.assert_allclose(dbi[j], getattr(m, f"bias_ih_l{l}{s}").grad.numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(dbh[j], getattr(m, f"bias_hh_l{l}{s}").grad.numpy(), rtol=0, atol=1e-12)


def pin_bwd_stack_bidirectional_finite_differences(orc):
    """Every gradient entry of a tiny two-direction two-layer stack against central differences of
    the pinned two-direction forward (lstm_stack_dirs)."""
    T, B, I, H, L = 3, 2, 2, 2, 2
    rng = np.random.default_rng(79)
    x = rng.normal(size=(T, B, I))
    Wi = [rng.normal(size=((I if j < 2 else 2 * H), 4 * H)) * 0.6 for j in range(2 * L)]
    Wh = [rng.normal(size=(H, 4 * H)) * 0.6 for _ in range(2 * L)]
    bi = [rng.normal(size=4 * H) * 0.3 for _ in range(2 * L)]
    bh = [rng.normal(size=4 * H) * 0.3 for _ in range(2 * L)]
    h0 = rng.normal(size=(2 * L, B, H)) * 0.5
    c0 = rng.normal(size=(2 * L, B, H)) * 0.5
    dout = rng.normal(size=(T, B, 2 * H))
    dhn = rng.normal(size=(2 * L, B, H))
    dcn = rng.normal(size=(2 * L, B, H))

    def loss():
        out, hn, cn = orc.lstm_stack_dirs(x, Wi, Wh, bi, bh, h0, c0, dirs=2)
        return float((out * dout).sum() + (hn * dhn).sum() + (cn * dcn).sum())

    grads = orc.lstm_stack_bwd(x, Wi, Wh, bi, bh, h0, c0, dout, dhn, dcn, dirs=2)
    targets = [(x, grads[0])] + list(zip(Wi, grads[1])) + list(zip(Wh, grads[2])) + list(zip(bi, grads[3])) + \
        list(zip(bh, grads[4])) + [(h0, grads[5]), (c0, grads[6])]
    eps = 1e-6
    for arr, g in targets:
        flat, gf = arr.reshape(-1), np.asarray(g).reshape(-1)
        for i in range(flat.size):
            v = flat[i]
            flat[i] = v + eps
            lp = loss()
            flat[i] = v - eps
            lm = loss()
            flat[i] = v
            assert abs((lp - lm) / (2 * eps) - gf[i]) <= 1e-7 * max(1.0, abs(gf[i])), (arr.shape, i)

ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
