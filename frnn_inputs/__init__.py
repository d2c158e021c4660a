"""Seeded synthetic inputs shared by the oracle side and the HIP side of every test and benchmark.

This module draws random numbers and nothing else: it holds none of the recurrence's arithmetic.
Both sides receive the identical stored tensors (same dtype, same bytes).

Recipe (the pages name no dataset; every input is synthetic):
* one CPU ``torch.Generator`` seeded with the workload's seed;
* draws in float32, in the fixed order Wx, R, b, states0 (stacked LSTM: x, then per layer
  Wi, Wh, b_ih, b_hh), then rounded to nearest-even into the stored dtype;
* ``N(0, v)`` names the variance v (std = sqrt(v)); ``U(a)`` is uniform on [-a, a).
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass, field
from typing import Optional, Tuple

import torch


@dataclass(frozen=True)
class HeadwiseWorkload:
    """A head-wise forward workload: Wx[B,T,G,N,D], R[G,N,D,D], b[G,N,D], states0[S,B,1,N,D]."""
    name: str
    cell: str            # "lstm" (G=4, S=2), "elman" (G=1, S=1) or "gru" (G=3, S=1)
    dtype: torch.dtype   # stored dtype of Wx, R, b, states0
    B: int
    T: int
    N: int
    D: int
    seed: int
    wx_var: float = 1.0
    r_var: Optional[float] = None      # None -> 1/D
    b_var: float = 0.1
    s0_var: Optional[float] = None     # None -> zero initial states (passed as NULL)

    @property
    def G(self) -> int:
        return {"lstm": 4, "elman": 1, "gru": 3}[self.cell]

    @property
    def S(self) -> int:
        return 2 if self.cell == "lstm" else 1


@dataclass(frozen=True)
class StackWorkload:
    """Plain multi-layer LSTM with input projection and one or two directions per layer: x[T,B,I],
    per layer and direction Wi[in,4H] (in = I, or dirs*H above layer 0), Wh[H,4H], b_ih, b_hh."""
    name: str
    dtype: torch.dtype
    L: int
    T: int
    B: int
    I: int
    H: int
    seed: int
    x_var: float = 1.0
    w_bound: Optional[float] = None    # None -> 1/sqrt(H)
    zero_init: bool = True
    dirs: int = 1


# The five workloads the recurrence is measured and checked on.
WORKLOADS = {
    "lstm_f32_B2_T16_N1_D32": HeadwiseWorkload(
        "lstm_f32_B2_T16_N1_D32", "lstm", torch.float32, B=2, T=16, N=1, D=32, seed=0, b_var=0.1),
    "lstm_bf16_B8_T1024_N3_D256": HeadwiseWorkload(
        "lstm_bf16_B8_T1024_N3_D256", "lstm", torch.bfloat16, B=8, T=1024, N=3, D=256, seed=1,
        b_var=1.0, s0_var=1.0),
    "lstm_bf16_B16_T1024_N1_D768": HeadwiseWorkload(
        "lstm_bf16_B16_T1024_N1_D768", "lstm", torch.bfloat16, B=16, T=1024, N=1, D=768, seed=2,
        b_var=0.1),
    "elman_bf16_B64_T2048_N12_D64": HeadwiseWorkload(
        "elman_bf16_B64_T2048_N12_D64", "elman", torch.bfloat16, B=64, T=2048, N=12, D=64, seed=3,
        b_var=0.1),
    "lstm2_bf16_T512_B32_I512_H512": StackWorkload(
        "lstm2_bf16_T512_B32_I512_H512", torch.bfloat16, L=2, T=512, B=32, I=512, H=512, seed=4),
}

HEADLINE = "lstm_bf16_B16_T1024_N1_D768"

# The two-layer LSTM workload's shape with both directions per layer (reading A21: the "5.3 LSTM"
# page's bidirectional flag and reverse weights): torch.nn.LSTM's init bound 1/sqrt(H).
BIDIR_WORKLOADS = {
    "lstm2bi_bf16_T512_B32_I512_H512": StackWorkload(
        "lstm2bi_bf16_T512_B32_I512_H512", torch.bfloat16, L=2, T=512, B=32, I=512, H=512, seed=5, dirs=2),
}

# The GRU cell (named in the FlashRNN cell list) on the shapes of the LSTM workloads above: the
# headline shape, the three-head shape with random initial state, and a small fp32 case.
GRU_WORKLOADS = {
    "gru_f32_B2_T16_N1_D32": HeadwiseWorkload(
        "gru_f32_B2_T16_N1_D32", "gru", torch.float32, B=2, T=16, N=1, D=32, seed=10, b_var=0.1,
        s0_var=0.25),
    "gru_bf16_B8_T1024_N3_D256": HeadwiseWorkload(
        "gru_bf16_B8_T1024_N3_D256", "gru", torch.bfloat16, B=8, T=1024, N=3, D=256, seed=11,
        b_var=1.0, s0_var=1.0),
    "gru_bf16_B16_T1024_N1_D768": HeadwiseWorkload(
        "gru_bf16_B16_T1024_N1_D768", "gru", torch.bfloat16, B=16, T=1024, N=1, D=768, seed=12,
        b_var=0.1),
}

# The headline shape with heads of 1024 units (the widest head the fused designs cover), LSTM and
# GRU.
WIDE_WORKLOADS = {
    "lstm_bf16_B16_T1024_N1_D1024": HeadwiseWorkload(
        "lstm_bf16_B16_T1024_N1_D1024", "lstm", torch.bfloat16, B=16, T=1024, N=1, D=1024, seed=13,
        b_var=0.1),
    "gru_bf16_B16_T1024_N1_D1024": HeadwiseWorkload(
        "gru_bf16_B16_T1024_N1_D1024", "gru", torch.bfloat16, B=16, T=1024, N=1, D=1024, seed=14,
        b_var=0.1),
}


def _normal(g: torch.Generator, shape, var: float) -> torch.Tensor:
    return torch.randn(shape, generator=g, dtype=torch.float32) * math.sqrt(var)


def _uniform(g: torch.Generator, shape, bound: float) -> torch.Tensor:
    return (torch.rand(shape, generator=g, dtype=torch.float32) * 2.0 - 1.0) * bound


def headwise_inputs(w: HeadwiseWorkload):
    """Return dict(Wx, R, b, states0) of CPU tensors in ``w.dtype`` (states0 may be None)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed)
    G, S, B, T, N, D = w.G, w.S, w.B, w.T, w.N, w.D
    r_var = (1.0 / D) if w.r_var is None else w.r_var
    Wx = _normal(g, (B, T, G, N, D), w.wx_var).to(w.dtype)
    R = _normal(g, (G, N, D, D), r_var).to(w.dtype)
    b = _normal(g, (G, N, D), w.b_var).to(w.dtype)
    s0 = None if w.s0_var is None else _normal(g, (S, B, 1, N, D), w.s0_var).to(w.dtype)
    return {"Wx": Wx, "R": R, "b": b, "states0": s0}


def backward_cotangents(w: HeadwiseWorkload):
    """Gradients of the forward's two outputs for a backward run: dstates [S,B,T,N,D] and dlast
    [S,B,1,N,D], float32 ~N(0,1), drawn in that order from a generator seeded with seed + 1000."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed + 1000)
    dstates = _normal(g, (w.S, w.B, w.T, w.N, w.D), 1.0)
    dlast = _normal(g, (w.S, w.B, 1, w.N, w.D), 1.0)
    return {"dstates": dstates, "dlast": dlast}


def stack_cotangents(w: StackWorkload):
    """Gradients of the multi-layer forward's outputs: dout [T,B,dirs*H], dhn and dcn [L*dirs,B,H],
    float32 ~N(0,1), drawn in that order from a generator seeded with seed + 1000."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed + 1000)
    dout = _normal(g, (w.T, w.B, w.dirs * w.H), 1.0)
    dhn = _normal(g, (w.L * w.dirs, w.B, w.H), 1.0)
    dcn = _normal(g, (w.L * w.dirs, w.B, w.H), 1.0)
    return {"dout": dout, "dhn": dhn, "dcn": dcn}


def stack_inputs(w: StackWorkload):
    """Return dict(x, Wi[], Wh[], b_ih[], b_hh[], h0, c0) of CPU tensors in ``w.dtype``; the weight
    lists hold L*dirs entries, layer l direction k at l*dirs + k, drawn in that order."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed)
    bound = (1.0 / math.sqrt(w.H)) if w.w_bound is None else w.w_bound
    x = _normal(g, (w.T, w.B, w.I), w.x_var).to(w.dtype)
    Wi, Wh, bih, bhh = [], [], [], []
    for l in range(w.L):
        for _ in range(w.dirs):
            fan_in = w.I if l == 0 else w.dirs * w.H
            Wi.append(_uniform(g, (fan_in, 4 * w.H), bound).to(w.dtype))
            Wh.append(_uniform(g, (w.H, 4 * w.H), bound).to(w.dtype))
            bih.append(_uniform(g, (4 * w.H,), bound).to(w.dtype))
            bhh.append(_uniform(g, (4 * w.H,), bound).to(w.dtype))
    h0 = c0 = None
    if not w.zero_init:
        h0 = _normal(g, (w.L * w.dirs, w.B, w.H), 1.0).to(w.dtype)
        c0 = _normal(g, (w.L * w.dirs, w.B, w.H), 1.0).to(w.dtype)
    return {"x": x, "Wi": Wi, "Wh": Wh, "b_ih": bih, "b_hh": bhh, "h0": h0, "c0": c0}


def get_workload(name: str):
    """A named workload from WORKLOADS, GRU_WORKLOADS, WIDE_WORKLOADS or BIDIR_WORKLOADS."""
    for table in (WORKLOADS, GRU_WORKLOADS, WIDE_WORKLOADS, BIDIR_WORKLOADS):
        if name in table:
            return table[name]
    raise KeyError(name)


def make_inputs(name_or_workload):
    w = get_workload(name_or_workload) if isinstance(name_or_workload, str) else name_or_workload
    if isinstance(w, HeadwiseWorkload):
        return headwise_inputs(w)
    return stack_inputs(w)


def sha256_of(t: Optional[torch.Tensor]) -> str:
    if t is None:
        return "none"
    return hashlib.sha256(t.contiguous().view(torch.uint8).numpy().tobytes()).hexdigest()


def to_f64(t: Optional[torch.Tensor]):
    """Exact widening of a stored tensor to a float64 numpy array (None passes through)."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()
