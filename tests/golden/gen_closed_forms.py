"""Write the golden fixtures in this folder from closed forms and hand-stepped scalar recurrences.

Independent of the oracle: everything here is evaluated with Python's ``decimal`` module at 50
significant digits, from the cell equations of "5.3 LSTM" (developnotes.readthedocs.io,
operator.html: i, f, o through a sigmoid, the cell input through tanh, c = f*c + i*g,
h = o*tanh(c)), the Elman cell h = tanh(Wx + r*h + b) of the FlashRNN cell list, and the textbook
GRU (named in that list, equations not printed). The pages print no numeric example of their own;
every value below is derived, and each file says how.

Run:  python tests/golden/gen_closed_forms.py
"""
from __future__ import annotations

import os
from decimal import Decimal, getcontext

getcontext().prec = 50
HERE = os.path.dirname(os.path.abspath(__file__))


def dexp(x: Decimal) -> Decimal:
    return x.exp()


def sig(x: Decimal) -> Decimal:
    return Decimal(1) / (Decimal(1) + dexp(-x))


def tanh(x: Decimal) -> Decimal:
    e2 = dexp(2 * x)
    return (e2 - 1) / (e2 + 1)


def fmt(v: Decimal) -> str:
    return format(v, ".25e")


def write(name: str, header: list[str], rows: dict[str, list[Decimal]]):
    path = os.path.join(HERE, name)
    with open(path, "w") as f:
        for line in header:
            f.write("# " + line + "\n")
        for key, vals in rows.items():
            f.write(key + " = " + " ".join(fmt(v) for v in vals) + "\n")
    print("wrote", path)


def lstm_const_pre(pre, c0: Decimal, T: int):
    """R = 0, constant pre-activations: c_t = f^t c0 + i z (1 - f^t) / (1 - f), h_t = o tanh(c_t)."""
    i, f, z, o = sig(pre[0]), sig(pre[1]), tanh(pre[2]), sig(pre[3])
    cs, hs = [], []
    for t in range(1, T + 1):
        ft = f ** t
        c = ft * c0 + i * z * (1 - ft) / (1 - f)
        cs.append(c)
        hs.append(o * tanh(c))
    return cs, hs


def main():
    # 1. pre = (0, 0, 1, 0), c0 = 0: f = i = o = 1/2, c_t = tanh(1) (1 - 2^-t), h_t = tanh(c_t)/2.
    T = 8
    cs, hs = lstm_const_pre([Decimal(0), Decimal(0), Decimal(1), Decimal(0)], Decimal(0), T)
    write("lstm_r0_pre_0010.txt", [
        "LSTM, one unit, R = 0, pre-activations constant over t: (i, f, z, o) = (0, 0, 1, 0), c0 = h0 = 0.",
        "Closed form of c = f*c + i*z with constant gates (geometric series): c_t = tanh(1)*(1 - 2^-t);",
        "h_t = o*tanh(c_t) = tanh(c_t)/2. Cell equations: 5.3 LSTM (developnotes, operator.html).",
        "Values for t = 1..8, 50-digit decimal arithmetic.",
    ], {"c": cs, "h": hs})

    # 2. general constant pre, nonzero c0, split as Wx + b (R = 0).
    wx = [Decimal("0.375"), Decimal("-0.5"), Decimal("1.25"), Decimal("0.625")]
    bb = [Decimal("-0.125"), Decimal("1.75"), Decimal("-0.25"), Decimal("0.5")]
    c0 = Decimal("-0.75")
    pre = [wx[g] + bb[g] for g in range(4)]
    cs, hs = lstm_const_pre(pre, c0, 12)
    write("lstm_r0_general.txt", [
        "LSTM, one unit, R = 0, Wx constant over t = (0.375, -0.5, 1.25, 0.625) for (i, f, z, o),",
        "b = (-0.125, 1.75, -0.25, 0.5), c0 = -0.75, h0 = 0 (h0 is irrelevant when R = 0).",
        "Closed form: c_t = f^t c0 + i z (1 - f^t)/(1 - f), h_t = o tanh(c_t), with",
        "i = sig(0.25), f = sig(1.25), z = tanh(1.0), o = sig(1.125). t = 1..12.",
        "Cell equations: 5.3 LSTM (developnotes, operator.html).",
    ], {"wx": wx, "b": bb, "c0": [c0], "c": cs, "h": hs})

    # 3. Elman, D = 1: h_t = tanh(1 + 0.5 h_{t-1}), h_0 = 0 (hand-stepped).
    h = Decimal(0)
    hs = []
    for _ in range(8):
        h = tanh(Decimal(1) + Decimal("0.5") * h)
        hs.append(h)
    write("elman_scalar.txt", [
        "Elman cell h = tanh(Wx + r*h + b) with D = 1, Wx = 1, r = 0.5, b = 0, h0 = 0, stepped by hand",
        "for t = 1..8 in 50-digit decimal arithmetic (cell named on the FlashRNN page; equation as",
        "stated for the Elman special case).",
    ], {"h": hs})

    # 4. Tiny LSTM, D = 2, T = 4, dense form of 5.3 LSTM: ifgo = x_t.Wi + h.Wh + bias with the
    #    pre-projected input given directly as xw_t (= x_t.Wi), Wh [2, 8] column blocks i, f, g, o.
    Wh = [[Decimal(v) for v in row] for row in (
        ["0.5", "-0.25", "0.75", "0.125", "-0.5", "1.0", "0.25", "-0.75"],
        ["-0.375", "0.625", "0.25", "-1.0", "0.875", "-0.125", "0.5", "0.375"],
    )]
    bias = [Decimal(v) for v in ["0.125", "-0.25", "0.5", "0.0", "-0.125", "0.375", "0.25", "-0.5"]]
    xw = [[Decimal(v) for v in row] for row in (
        ["1.0", "-0.5", "0.25", "0.75", "-1.25", "0.5", "0.125", "-0.375"],
        ["-0.625", "0.875", "-0.25", "0.5", "1.5", "-0.75", "0.375", "0.25"],
        ["0.25", "0.125", "-1.0", "-0.5", "0.5", "1.25", "-0.875", "0.625"],
        ["0.75", "-1.5", "0.5", "0.25", "-0.25", "0.0", "1.0", "-0.125"],
    )]
    h = [Decimal("0.25"), Decimal("-0.5")]
    c = [Decimal("0.5"), Decimal("-1.0")]
    hs, cs = [], []
    for t in range(4):
        ifgo = [xw[t][j] + sum(h[k] * Wh[k][j] for k in range(2)) + bias[j] for j in range(8)]
        newc, newh = [], []
        for e in range(2):
            i_ = sig(ifgo[0 + e]); f_ = sig(ifgo[2 + e]); g_ = tanh(ifgo[4 + e]); o_ = sig(ifgo[6 + e])
            ce = f_ * c[e] + i_ * g_
            newc.append(ce)
            newh.append(o_ * tanh(ce))
        c, h = newc, newh
        hs.extend(h)
        cs.extend(c)
    flat_wh = [v for row in Wh for v in row]
    flat_xw = [v for row in xw for v in row]
    write("lstm_tiny_d2_t4.txt", [
        "LSTM, B = 1, one head, D = 2, T = 4, hand-stepped in the dense form of 5.3 LSTM",
        "(developnotes, operator.html): ifgo = xw_t + h.Wh + bias, Wh stored [H, 4H] with column",
        "blocks i | f | g | o, h0 = (0.25, -0.5), c0 = (0.5, -1.0). xw rows are t = 0..3 (already",
        "projected input, 8 columns). Outputs h, c listed t-major: h[t=1][0], h[t=1][1], h[t=2][0] ...",
    ], {"wh": flat_wh, "bias": bias, "xw": flat_xw, "h0": [Decimal("0.25"), Decimal("-0.5")],
        "c0": [Decimal("0.5"), Decimal("-1.0")], "h": hs, "c": cs})

    # 5. GRU, D = 1, nonzero recurrent weights, hand-stepped: r = sig(wx_r + R_r h + b_r),
    #    z = sig(wx_z + R_z h + b_z), n = tanh(wx_n + r (R_n h + b_n)), h' = (1 - z) n + z h.
    gwx = [Decimal("0.5"), Decimal("-0.25"), Decimal("0.75")]
    gR = [Decimal("0.5"), Decimal("-0.75"), Decimal("1.25")]
    gb = [Decimal("0.125"), Decimal("0.25"), Decimal("-0.5")]
    h = Decimal("-0.5")
    hs = []
    for _ in range(8):
        r = sig(gwx[0] + gR[0] * h + gb[0])
        z = sig(gwx[1] + gR[1] * h + gb[1])
        n = tanh(gwx[2] + r * (gR[2] * h + gb[2]))
        h = (1 - z) * n + z * h
        hs.append(h)
    write("gru_scalar.txt", [
        "GRU, one unit, stepped by hand for t = 1..8 in 50-digit decimal arithmetic, in the textbook",
        "form whose reset gate scales the recurrent part of the candidate after the product:",
        "r = sig(wx_r + R_r h + b_r), z = sig(wx_z + R_z h + b_z), n = tanh(wx_n + r (R_n h + b_n)),",
        "h' = (1 - z) n + z h. Gate order r, z, n; wx constant over t; h0 = -0.5. (The FlashRNN page",
        "names the GRU among its cells without printing its equations.)",
    ], {"wx": gwx, "r": gR, "b": gb, "h0": [Decimal("-0.5")], "h": hs})


if __name__ == "__main__":
    main()
