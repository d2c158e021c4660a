"""fp64 CPU oracle for the head-wise LSTM / Elman forward recurrence and the plain multi-layer LSTM.

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the benchmark's CPU-baseline leg may
use this package; the product path (``head_wise_lstm_amd``) never imports, loads or calls it, and
this package imports nothing from the product.

The arithmetic lives in ``frnn_oracle.c`` (plain C, double precision, OpenMP over independent
(batch, head) rows); this module only marshals numpy float64 arrays to it. What is computed:

* ``headwise_fwd`` -- FlashRNN usage example (hottg.com/neural/9889): layouts Wx[B,T,G,N,D],
  R[G,N,D,D], b[G,N,D], states[S,B,T,N,D], last_states[S,B,1,N,D]; the cell is the one of
  "5.3 LSTM" (developnotes.readthedocs.io, operator.html) applied per head, gates i, f, z, o along
  G; Elman: h = tanh(Wx + h.R + b); GRU (named in the FlashRNN cell list, equations not printed):
  the textbook cell with gates r, z, n along G, the reset gate scaling the candidate's recurrent
  part h.R_n + b_n, h' = (1 - z) n + z h, S = 1.
* ``headwise_bwd`` -- back-propagation through time of ``headwise_fwd``: the gradients of
  sum(dstates * states) + sum(dlast * last_states) with respect to Wx, R, b and states0. The pages
  print no gradient formulas; the C source writes out the chain rule of the cell equations.
* ``lstm_stack_bwd`` -- the gradients of the multi-layer LSTM (one or two directions per layer),
  composed layer by layer of the pinned head-wise forward and backward and library matmuls for the
  projections.
* ``lstm_stack_p3`` -- "5.3 LSTM", MyLSTM.set_weights and MyLSTM.forward: time loop outermost,
  layers inside it, bias = bias_ih + bias_hh, Wi stored [in, 4H], Wh stored [H, 4H].
* ``lstm_stack_dirs`` -- the same cell with one or two directions per layer, layer by layer. The
  page's MyLSTM takes ``bidirectional`` and copies "_reverse" weights but its forward never uses
  them; the reading (torch.nn.LSTM's): direction 1 runs the layer's input from the last step to
  the first with its own weights, and a layer's output is [h of direction 0, h of direction 1].

Pins (tests/test_oracle_pins.py): closed forms (R = 0 geometric gating, saturated forget gate,
Elman and GRU scalar iterations) computed independently at 50 significant digits, GRU closed forms
(R = 0, saturated update gate, shut reset gate), torch.nn.LSTM / nn.RNN / nn.GRU in float64 as
library special cases, head / batch / continuation invariants, and hand-stepped tiny cases. The
backward: torch autograd through float64 torch.nn.LSTM / GRU / RNN layers with identity input
weights (so that their input is Wx), central finite differences of the pinned forward on every
entry, linearity in the cotangent, and T = 0.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "frnn_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

CELL_LSTM = 0
CELL_ELMAN = 1
CELL_GRU = 2


def build(verbose: bool = False, source: str = SOURCE, out: str = LIB_PATH) -> str:
    """Compile the oracle with gcc (IEEE double, no fast-math) into a shared library."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", source, "-o", out, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return out


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


class Oracle:
    """ctypes front of one compiled copy of frnn_oracle.c."""

    def __init__(self, lib_path: str = LIB_PATH):
        if not os.path.exists(lib_path):
            if lib_path != LIB_PATH:
                raise FileNotFoundError(lib_path)
            build()
        lib = ctypes.CDLL(lib_path)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.oracle_headwise_fwd.restype = ctypes.c_int
        lib.oracle_headwise_fwd.argtypes = [
            ctypes.c_int, ctypes.c_long, ctypes.c_long, ctypes.c_long, ctypes.c_long,
            dp, dp, dp, dp, dp, dp, ctypes.POINTER(ctypes.c_long), ctypes.c_long,
        ]
        lib.oracle_headwise_bwd.restype = ctypes.c_int
        lib.oracle_headwise_bwd.argtypes = [
            ctypes.c_int, ctypes.c_long, ctypes.c_long, ctypes.c_long, ctypes.c_long,
            dp, dp, dp, dp, dp, dp, dp, dp, dp, dp,
        ]
        lib.oracle_lstm_stack_p3.restype = ctypes.c_int
        lib.oracle_lstm_stack_p3.argtypes = [
            ctypes.c_long, ctypes.c_long, ctypes.c_long, ctypes.c_long, ctypes.c_long,
            dp, ctypes.POINTER(dp), ctypes.POINTER(dp), ctypes.POINTER(dp), ctypes.POINTER(dp),
            dp, dp, dp, dp, dp,
        ]
        lib.oracle_lstm_stack_dirs.restype = ctypes.c_int
        lib.oracle_lstm_stack_dirs.argtypes = [
            ctypes.c_long, ctypes.c_long, ctypes.c_long, ctypes.c_long, ctypes.c_long, ctypes.c_long,
            dp, ctypes.POINTER(dp), ctypes.POINTER(dp), ctypes.POINTER(dp), ctypes.POINTER(dp),
            dp, dp, dp, dp, dp,
        ]
        self.lib = lib

    def headwise_fwd(self, cell: str, Wx, R, b, states0=None, pairs=None, want_states: bool = True):
        """Head-wise forward in float64.

        Wx [B,T,G,N,D], R [G,N,D,D], b [G,N,D] (None = zeros), states0 [S,B,1,N,D] or None
        (zeros). ``pairs``: optional iterable of flattened (b*N + n) rows to compute (the others
        stay NaN). Returns (states [S,B,T,N,D] or None, last_states [S,B,1,N,D]).
        """
        c = {"lstm": CELL_LSTM, "elman": CELL_ELMAN, "gru": CELL_GRU}[cell]
        G, S = {CELL_LSTM: (4, 2), CELL_ELMAN: (1, 1), CELL_GRU: (3, 1)}[c]
        Wx, R = _f64(Wx), _f64(R)
        B, T, G_, N, D = Wx.shape
        b = np.zeros((G, N, D)) if b is None else _f64(b)
        states0 = _f64(states0)
        if G_ != G or R.shape != (G, N, D, D) or b.shape != (G, N, D):
            raise ValueError("shape mismatch")
        if states0 is not None and states0.shape != (S, B, 1, N, D):
            raise ValueError("states0 shape mismatch")
        states = np.full((S, B, T, N, D), np.nan) if want_states else None
        last = np.full((S, B, 1, N, D), np.nan)
        if pairs is not None:
            pr = np.ascontiguousarray(np.asarray(list(pairs), dtype=np.int64))
            pp, npairs = pr.ctypes.data_as(ctypes.POINTER(ctypes.c_long)), len(pr)
        else:
            pr, pp, npairs = None, None, 0
        rc = self.lib.oracle_headwise_fwd(c, B, T, N, D, _ptr(Wx), _ptr(R), _ptr(b), _ptr(states0),
                                          _ptr(states), _ptr(last), pp, npairs)
        if rc != 0:
            raise RuntimeError("oracle_headwise_fwd failed")
        return states, last

    def headwise_bwd(self, cell: str, Wx, R, b, states0=None, dstates=None, dlast=None):
        """Head-wise backward in float64: the gradients of L = sum(dstates * states) +
        sum(dlast * last_states) with respect to the forward's inputs.

        Same inputs as headwise_fwd, plus dstates [S,B,T,N,D] and dlast [S,B,1,N,D] (None =
        zeros). Returns (dWx [B,T,G,N,D], dR [G,N,D,D], db [G,N,D], dstates0 [S,B,1,N,D]).
        """
        c = {"lstm": CELL_LSTM, "elman": CELL_ELMAN, "gru": CELL_GRU}[cell]
        G, S = {CELL_LSTM: (4, 2), CELL_ELMAN: (1, 1), CELL_GRU: (3, 1)}[c]
        Wx, R = _f64(Wx), _f64(R)
        B, T, G_, N, D = Wx.shape
        b = np.zeros((G, N, D)) if b is None else _f64(b)
        states0, dstates, dlast = _f64(states0), _f64(dstates), _f64(dlast)
        if G_ != G or R.shape != (G, N, D, D) or b.shape != (G, N, D):
            raise ValueError("shape mismatch")
        for name, a, shp in (("states0", states0, (S, B, 1, N, D)), ("dstates", dstates, (S, B, T, N, D)),
                             ("dlast", dlast, (S, B, 1, N, D))):
            if a is not None and a.shape != shp:
                raise ValueError(f"{name} shape mismatch")
        dWx = np.empty((B, T, G, N, D))
        dR = np.empty((G, N, D, D))
        db = np.empty((G, N, D))
        ds0 = np.empty((S, B, 1, N, D))
        rc = self.lib.oracle_headwise_bwd(c, B, T, N, D, _ptr(Wx), _ptr(R), _ptr(b), _ptr(states0),
                                          _ptr(dstates), _ptr(dlast), _ptr(dWx), _ptr(dR), _ptr(db),
                                          _ptr(ds0))
        if rc != 0:
            raise RuntimeError("oracle_headwise_bwd failed")
        return dWx, dR, db, ds0

    def lstm_stack_p3(self, x, Wi, Wh, b_ih, b_hh, h0=None, c0=None):
        """Plain multi-layer LSTM of "5.3 LSTM" in float64.

        x [T,B,I]; Wi, Wh, b_ih, b_hh: lists over layers ([in,4H], [H,4H], [4H], [4H]; a bias
        may be None = zeros); h0, c0 [L,B,H] or None. Returns (out [T,B,H], hn, cn [L,B,H]).
        """
        x = _f64(x)
        T, B, I = x.shape
        L = len(Wi)
        H = Wh[0].shape[0]
        Wi = [_f64(w) for w in Wi]
        Wh = [_f64(w) for w in Wh]
        b_ih = [np.zeros(4 * H) if v is None else _f64(v) for v in b_ih]
        b_hh = [np.zeros(4 * H) if v is None else _f64(v) for v in b_hh]
        for l in range(L):
            if Wi[l].shape != ((I if l == 0 else H), 4 * H) or Wh[l].shape != (H, 4 * H):
                raise ValueError("weight shape mismatch")
        h0, c0 = _f64(h0), _f64(c0)
        out = np.empty((T, B, H))
        hn = np.empty((L, B, H))
        cn = np.empty((L, B, H))
        arr = ctypes.POINTER(ctypes.c_double) * L
        rc = self.lib.oracle_lstm_stack_p3(
            L, T, B, I, H, _ptr(x), arr(*[_ptr(w) for w in Wi]), arr(*[_ptr(w) for w in Wh]),
            arr(*[_ptr(v) for v in b_ih]), arr(*[_ptr(v) for v in b_hh]), _ptr(h0), _ptr(c0),
            _ptr(out), _ptr(hn), _ptr(cn))
        if rc != 0:
            raise RuntimeError("oracle_lstm_stack_p3 failed")
        return out, hn, cn


    def lstm_stack_dirs(self, x, Wi, Wh, b_ih, b_hh, h0=None, c0=None, dirs: int = 1):
        """Multi-layer LSTM with ``dirs`` (1 or 2) directions per layer, in float64.

        x [T,B,I]; Wi, Wh, b_ih, b_hh: lists of L*dirs entries, layer l direction k at l*dirs + k
        ([in,4H] with in = I for l = 0 else dirs*H, [H,4H], [4H], [4H]; a bias may be None);
        h0, c0 [L*dirs,B,H] or None. Returns (out [T,B,dirs*H], hn, cn [L*dirs,B,H]).
        """
        x = _f64(x)
        T, B, I = x.shape
        if dirs not in (1, 2) or len(Wi) % dirs:
            raise ValueError("dirs must be 1 or 2, with dirs weights per layer")
        L = len(Wi) // dirs
        H = Wh[0].shape[0]
        Wi = [_f64(w) for w in Wi]
        Wh = [_f64(w) for w in Wh]
        b_ih = [np.zeros(4 * H) if v is None else _f64(v) for v in b_ih]
        b_hh = [np.zeros(4 * H) if v is None else _f64(v) for v in b_hh]
        for j in range(L * dirs):
            if Wi[j].shape != ((I if j < dirs else dirs * H), 4 * H) or Wh[j].shape != (H, 4 * H):
                raise ValueError("weight shape mismatch")
        h0, c0 = _f64(h0), _f64(c0)
        out = np.empty((T, B, dirs * H))
        hn = np.empty((L * dirs, B, H))
        cn = np.empty((L * dirs, B, H))
        arr = ctypes.POINTER(ctypes.c_double) * (L * dirs)
        rc = self.lib.oracle_lstm_stack_dirs(
            L, dirs, T, B, I, H, _ptr(x), arr(*[_ptr(w) for w in Wi]), arr(*[_ptr(w) for w in Wh]),
            arr(*[_ptr(v) for v in b_ih]), arr(*[_ptr(v) for v in b_hh]), _ptr(h0), _ptr(c0),
            _ptr(out), _ptr(hn), _ptr(cn))
        if rc != 0:
            raise RuntimeError("oracle_lstm_stack_dirs failed")
        return out, hn, cn

    def lstm_stack_bwd(self, x, Wi, Wh, b_ih, b_hh, h0=None, c0=None, dout=None, dhn=None, dcn=None,
                       dirs: int = 1):
        """Backward of the multi-layer LSTM (``dirs`` = 1: "5.3 LSTM"; 2: reading A21's two
        directions per layer) in float64: the gradients of L = sum(dout * out) + sum(dhn * hn) +
        sum(dcn * cn) with respect to x, Wi[j], Wh[j], b_ih[j], b_hh[j], h0 and c0, with j = l * dirs
        + k for layer l, direction k (shapes as for lstm_stack_dirs).

        Composed of steps already pinned on their own, layer by layer (layer-major order, equal to the
        page's time-major loop; reading A13): per layer and direction, the projection Wx = X.Wi + b_ih
        + b_hh (a library matmul) of the layer's input X in the direction's own time order (direction
        1 takes the sequence from the last step to the first), the head-wise forward and backward
        (headwise_fwd / headwise_bwd with R[g,0,d,e] = Wh[d, g*H + e]), then dWi = X^T.dWx,
        db_ih = db_hh = sum dWx, and the direction's part of dX = dWx.Wi^T, put back in time order;
        the layer's dX is the sum over its directions. The layer output's gradient for direction k
        is columns k*H .. k*H + H - 1 of the gradient reaching it. Returns (dx, dWi[], dWh[],
        db_ih[], db_hh[], dh0, dc0).
        """
        x = _f64(x)
        T, B, I = x.shape
        if dirs not in (1, 2) or len(Wi) % dirs:
            raise ValueError("dirs must be 1 or 2, with dirs weights per layer")
        L = len(Wi) // dirs
        H = Wh[0].shape[0]
        J = L * dirs
        Wi = [_f64(w) for w in Wi]
        Wh = [_f64(w) for w in Wh]
        b_ih = [np.zeros(4 * H) if v is None else _f64(v) for v in b_ih]
        b_hh = [np.zeros(4 * H) if v is None else _f64(v) for v in b_hh]
        h0 = np.zeros((J, B, H)) if h0 is None else _f64(h0)
        c0 = np.zeros((J, B, H)) if c0 is None else _f64(c0)

        def order(a, k):  # a [T, ...] in direction k's time order (and back: the map is its own inverse)
            return a if k == 0 else a[::-1]

        # forward, keeping every layer's input sequence and every direction's projection
        X, Wxs, Rs, s0s = [x], [None] * J, [None] * J, [None] * J
        for l in range(L):
            outs = []
            for k in range(dirs):
                j = l * dirs + k
                proj = order(X[l], k) @ Wi[j] + (b_ih[j] + b_hh[j])          # [T,B,4H], own time order
                Wxs[j] = proj.reshape(T, B, 4, 1, H).transpose(1, 0, 2, 3, 4)  # [B,T,4,1,H]
                Rs[j] = Wh[j].reshape(H, 4, H).transpose(1, 0, 2)[:, None]      # R[g,0,d,e] = Wh[d, gH+e]
                s0s[j] = np.stack([h0[j], c0[j]])[:, :, None, None, :]         # [2,B,1,1,H]
                st, _ = self.headwise_fwd("lstm", Wxs[j], Rs[j], None, s0s[j])
                outs.append(order(st[0, :, :, 0].transpose(1, 0, 2), k))      # [T,B,H] in time order
            X.append(np.concatenate(outs, axis=2))                           # [T,B,dirs*H]
        dX = np.zeros((T, B, dirs * H)) if dout is None else _f64(dout)
        dWi, dWh, dbi, dbh = [None] * J, [None] * J, [None] * J, [None] * J
        dh0, dc0 = np.zeros((J, B, H)), np.zeros((J, B, H))
        for l in range(L - 1, -1, -1):
            dXin = np.zeros(X[l].shape)
            for k in range(dirs):
                j = l * dirs + k
                dstates = np.zeros((2, B, T, 1, H))
                dstates[0, :, :, 0] = order(dX[:, :, k * H:(k + 1) * H], k).transpose(1, 0, 2)
                dlast = np.zeros((2, B, 1, 1, H))
                if dhn is not None:
                    dlast[0, :, 0, 0] = _f64(dhn)[j]
                if dcn is not None:
                    dlast[1, :, 0, 0] = _f64(dcn)[j]
                dWx, dR, _, ds0 = self.headwise_bwd("lstm", Wxs[j], Rs[j], None, s0s[j], dstates, dlast)
                dproj = dWx[:, :, :, 0].transpose(1, 0, 2, 3).reshape(T, B, 4 * H)  # [T,B,4H], own order
                dWh[j] = dR[:, 0].transpose(1, 0, 2).reshape(H, 4 * H)            # dWh[d, gH+e] = dR[g,0,d,e]
                Xk = order(X[l], k)
                dWi[j] = Xk.reshape(T * B, -1).T @ dproj.reshape(T * B, 4 * H)
                dbi[j] = dproj.reshape(T * B, 4 * H).sum(axis=0)
                dbh[j] = dbi[j].copy()
                dh0[j], dc0[j] = ds0[0, :, 0, 0], ds0[1, :, 0, 0]
                dXin += order(dproj @ Wi[j].T, k)                                 # [T,B,in], time order
            dX = dXin
        return dX, dWi, dWh, dbi, dbh, dh0, dc0


def lstm_stack_bwd(orc, *args, **kwargs):
    """``orc.lstm_stack_bwd(...)`` (kept as a function for callers that pass the oracle)."""
    return orc.lstm_stack_bwd(*args, **kwargs)


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def headwise_fwd(*args, **kwargs):
    return default().headwise_fwd(*args, **kwargs)


def headwise_bwd(*args, **kwargs):
    return default().headwise_bwd(*args, **kwargs)


def lstm_stack_p3(*args, **kwargs):
    return default().lstm_stack_p3(*args, **kwargs)


def lstm_stack_dirs(*args, **kwargs):
    return default().lstm_stack_dirs(*args, **kwargs)


def lstm_stack_bwd_p3(*args, **kwargs):
    return lstm_stack_bwd(default(), *args, **kwargs)
