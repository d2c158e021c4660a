"""HIP backward (frnn_bwd) against the fp64 oracle's back-propagation through time.

The GPU runs its own forward, then the backward from the states it returned; the oracle runs
both in fp64 on the same stored inputs and the same seeded cotangents (dstates, dlast ~ N(0,1)).

Bar, per gradient tensor X (dWx, dR, db, dstates0): max|X_gpu - X_oracle| <= tol * max(1,
max|X_oracle|), relative to the tensor's scale because dR and db are sums over all B*T steps and
grow with them. tol = 1e-2 for bf16 inputs: the contractions take bf16 copies of h and of the
gradient of the gate pre-activations (unit roundoff 2^-9, about 2e-3, on each operand), so an
element carries a few units of it relative to the largest element; 1e-2 is five. tol = 1e-5 for
fp32 inputs, a few hundred fp32 units for sums over up to B*T*D terms.
"""
import ctypes
import os
import sys

import numpy as np
import pytest
import torch

import frnn_inputs as fi
import oracle

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-5, torch.bfloat16: 1e-2}


def _hw():
    import head_wise_lstm_amd as hw
    return hw


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    _hw().load()


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class _env:
    """Set environment variables (planner overrides) for the duration of a block."""

    def __init__(self, env):
        self.env = {k: str(v) for k, v in (env or {}).items()}

    def __enter__(self):
        self.old = {k: os.environ.get(k) for k in self.env}
        os.environ.update(self.env)

    def __exit__(self, *exc):
        for k, v in self.old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def run_bwd_case(w, path="alternating", env=None):
    with _env(env):
        return _run_bwd_case(w, path)


def _run_bwd_case(w, path):
    hw = _hw()
    x = fi.make_inputs(w)
    ct = fi.backward_cotangents(w)
    dev = torch.device("cuda:0")
    g = lambda t: None if t is None else t.to(dev)
    _log(f"bwd case {w.name} cell={w.cell} B={w.B} T={w.T} N={w.N} D={w.D} path={path}")
    if path == "fused":
        _log("  plan: " + hw.frnn_bwd_plan_str(hw._desc(w.B, w.T, w.N, w.D, w.cell, w.dtype), "fused"))
    try:  # the forward on the fused path where it has a design
        hw.frnn_plan_str(hw._desc(w.B, w.T, w.N, w.D, w.cell, w.dtype), "fused")
        fwd_path = "fused"
    except hw.FrnnError:
        fwd_path = "alternating"
    st, last = hw.frnn_fwd(g(x["Wx"]), g(x["R"]), g(x["b"]), g(x["states0"]), cell=w.cell, path=fwd_path)
    grads = hw.frnn_bwd(g(x["Wx"]), g(x["R"]), g(x["b"]), g(x["states0"]), st, g(ct["dstates"]), g(ct["dlast"]),
                        cell=w.cell, path=path)
    torch.cuda.synchronize()
    f = fi.to_f64
    ref = oracle.headwise_bwd(w.cell, f(x["Wx"]), f(x["R"]), f(x["b"]), f(x["states0"]), f(ct["dstates"]),
                              f(ct["dlast"]))
    tol = TOL[w.dtype]
    errs = {}
    for name, gv, rv in zip(("dWx", "dR", "db", "dstates0"), grads, ref):
        gv = gv.double().cpu().numpy()
        assert gv.shape == rv.shape, name
        assert np.all(np.isfinite(gv)), name
        scale = max(1.0, float(np.abs(rv).max())) if rv.size else 1.0
        err = float(np.abs(gv - rv).max()) if rv.size else 0.0
        errs[name] = (err, scale)
    _log("  " + " ".join(f"{k}: err={e:.3e} scale={s:.3g} rel={e / s:.2e}" for k, (e, s) in errs.items()))
    for k, (e, s) in errs.items():
        assert e <= tol * s, f"{k}: max abs err {e} > {tol} * {s}"
    return errs


SMALL = [
    fi.HeadwiseWorkload("bwd_lstm_bf16_ragged_D64", "lstm", torch.bfloat16, B=5, T=13, N=2, D=64, seed=201, s0_var=1.0),
    fi.HeadwiseWorkload("bwd_lstm_bf16_D96", "lstm", torch.bfloat16, B=19, T=7, N=2, D=96, seed=202, s0_var=0.5),
    fi.HeadwiseWorkload("bwd_lstm_bf16_D256", "lstm", torch.bfloat16, B=9, T=12, N=2, D=256, seed=203, s0_var=1.0,
                        b_var=1.0),
    fi.HeadwiseWorkload("bwd_elman_bf16_D64", "elman", torch.bfloat16, B=21, T=9, N=3, D=64, seed=204, s0_var=1.0),
    fi.HeadwiseWorkload("bwd_elman_bf16_D128", "elman", torch.bfloat16, B=7, T=10, N=2, D=128, seed=205),
    fi.HeadwiseWorkload("bwd_gru_bf16_D64", "gru", torch.bfloat16, B=5, T=13, N=2, D=64, seed=206, s0_var=1.0),
    fi.HeadwiseWorkload("bwd_gru_bf16_D256", "gru", torch.bfloat16, B=9, T=12, N=2, D=256, seed=207, s0_var=1.0,
                        b_var=1.0),
    fi.HeadwiseWorkload("bwd_lstm_f32_D32", "lstm", torch.float32, B=3, T=11, N=2, D=32, seed=208, s0_var=1.0),
    fi.HeadwiseWorkload("bwd_elman_f32_D64", "elman", torch.float32, B=4, T=9, N=3, D=64, seed=209, s0_var=1.0),
    fi.HeadwiseWorkload("bwd_gru_f32_D32", "gru", torch.float32, B=3, T=11, N=2, D=32, seed=210, s0_var=1.0),
    fi.HeadwiseWorkload("bwd_lstm_bf16_T1", "lstm", torch.bfloat16, B=1, T=1, N=1, D=64, seed=211, s0_var=1.0),
    # 32-unit Elman heads on the single-workgroup design: eight rows a workgroup (compact records),
    # the second group of each head ragged (three rows)
    fi.HeadwiseWorkload("bwd_elman_bf16_D32", "elman", torch.bfloat16, B=11, T=10, N=2, D=32, seed=212, s0_var=1.0),
    fi.HeadwiseWorkload("bwd_elman_f32_D32", "elman", torch.float32, B=11, T=7, N=2, D=32, seed=213, s0_var=1.0),
]


def _fused_plan_or_skip(w):
    hw = _hw()
    try:
        return hw.frnn_bwd_plan_str(hw._desc(w.B, w.T, w.N, w.D, w.cell, w.dtype), "fused")
    except hw.FrnnError as e:
        if e.status == -2:
            pytest.skip("no fused backward design for this shape or dtype (fp32, or no die-local tiling)")
        raise


@pytest.mark.parametrize("path", ["alternating", "fused"])
@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_bwd_small(w, path):
    if path == "fused":
        _fused_plan_or_skip(w)
    run_bwd_case(w, path)


@pytest.mark.parametrize("path", ["alternating", "fused"])
@pytest.mark.parametrize("name", ["lstm_bf16_B16_T1024_N1_D768", "lstm_bf16_B8_T1024_N3_D256",
                                  "gru_bf16_B16_T1024_N1_D768", "lstm_f32_B2_T16_N1_D32",
                                  "elman_bf16_B64_T2048_N12_D64"])
def test_bwd_full(name, path):
    w = fi.get_workload(name)
    if path == "fused":
        _fused_plan_or_skip(w)
    run_bwd_case(w, path)


# Both forms of the alternating backward's step, pinned with FRNN_ALT_BWD_ONE_LAUNCH: one launch
# (the contraction with the step's gradients as its epilogue; the choice for G*D <= 1024) and two
# (the gradients, then the K-split contraction).
@pytest.mark.parametrize("one", [1, 0])
@pytest.mark.parametrize("w", [x for x in SMALL if x.name in ("bwd_lstm_bf16_ragged_D64", "bwd_gru_bf16_D256",
                                                                "bwd_elman_bf16_D128", "bwd_lstm_f32_D32")],
                         ids=lambda w: w.name)
def test_bwd_alternating_each_form(w, one):
    hw = _hw()
    with _env({"FRNN_ALT_BWD_ONE_LAUNCH": one}):
        plan = hw.frnn_bwd_plan_str(hw._desc(w.B, w.T, w.N, w.D, w.cell, w.dtype), "alternating")
    assert f"step_launches={w.T if one else 2 * w.T}" in plan, plan
    run_bwd_case(w, "alternating", env={"FRNN_ALT_BWD_ONE_LAUNCH": one})


# Every fused backward design on the small bf16 cases, pinned with FRNN_FUSED_BWD_PX: the
# partial-sum design (the planner's choice for heads wider than 64 units), the da-exchange design,
# and, for heads of at most 64 units, the single-workgroup design (the planner's choice there).
# Heads of 32 units have only the last.
_DESIGN_NAME = {1: "die-local-partials", 0: "design=die-local ", 2: "workgroup-local"}


@pytest.mark.parametrize("w,px", [(x, px) for x in SMALL if x.dtype == torch.bfloat16 for px in (1, 0, 2)
                                  if (px != 2 or x.D <= 64) and (px == 2 or x.D > 32)],
                         ids=lambda x: f"px{x}" if isinstance(x, int) else x.name)
def test_bwd_small_each_design(w, px):
    with _env({"FRNN_FUSED_BWD_PX": px}):
        plan = _fused_plan_or_skip(w)
    assert _DESIGN_NAME[px] in plan + " ", plan
    run_bwd_case(w, "fused", env={"FRNN_FUSED_BWD_PX": px})


# The partial-sum design forced onto shapes and splits the planner would not pick: several rows
# per group, a ragged last block, units per workgroup from 8 to 64, every cell.
PX_FORCED = [
    (fi.HeadwiseWorkload("px_lstm_D256_W16_BR4", "lstm", torch.bfloat16, B=7, T=9, N=2, D=256, seed=281, s0_var=1.0),
     {"FRNN_FUSED_BWD_W": 16, "FRNN_FUSED_BWD_BR": 4}),
    (fi.HeadwiseWorkload("px_lstm_D768_BR3", "lstm", torch.bfloat16, B=7, T=6, N=1, D=768, seed=282, s0_var=1.0),
     {"FRNN_FUSED_BWD_W": 32, "FRNN_FUSED_BWD_BR": 3}),
    (fi.HeadwiseWorkload("px_lstm_D128_W16", "lstm", torch.bfloat16, B=5, T=8, N=2, D=128, seed=283, s0_var=1.0),
     {"FRNN_FUSED_BWD_W": 16, "FRNN_FUSED_BWD_BR": 2}),
    (fi.HeadwiseWorkload("px_lstm_D768_6waves", "lstm", torch.bfloat16, B=4, T=7, N=1, D=768, seed=284, s0_var=1.0),
     {"FRNN_FUSED_BWD_W": 32, "FRNN_FUSED_BWD_NCW": 6}),
    (fi.HeadwiseWorkload("px_gru_D256_W8_BR3", "gru", torch.bfloat16, B=8, T=9, N=2, D=256, seed=285, s0_var=1.0),
     {"FRNN_FUSED_BWD_W": 8, "FRNN_FUSED_BWD_BR": 3}),
    (fi.HeadwiseWorkload("px_elman_D128_W2", "elman", torch.bfloat16, B=5, T=10, N=2, D=128, seed=286, s0_var=1.0),
     {"FRNN_FUSED_BWD_W": 2, "FRNN_FUSED_BWD_BR": 2}),
    (fi.HeadwiseWorkload("px_elman_D768", "elman", torch.bfloat16, B=6, T=8, N=1, D=768, seed=287, s0_var=1.0),
     {"FRNN_FUSED_BWD_W": 24, "FRNN_FUSED_BWD_BR": 3}),
]


@pytest.mark.parametrize("w,env", PX_FORCED, ids=lambda x: getattr(x, "name", ""))
def test_bwd_partials_forced(w, env):
    env = dict(env, FRNN_FUSED_BWD_PX=1)
    with _env(env):
        plan = _fused_plan_or_skip(w)
    assert "die-local-partials" in plan and f"W={env['FRNN_FUSED_BWD_W']} " in plan, plan
    run_bwd_case(w, "fused", env=env)


# Extreme shapes (as in the forward tests): D = 1024, many narrow heads, wide batches.
BWD_EXTREME = [
    fi.HeadwiseWorkload("bwd_lstm_D1024", "lstm", torch.bfloat16, B=2, T=6, N=1, D=1024, seed=301, s0_var=1.0),
    fi.HeadwiseWorkload("bwd_gru_D1024", "gru", torch.bfloat16, B=3, T=5, N=1, D=1024, seed=302, s0_var=1.0),
    fi.HeadwiseWorkload("bwd_lstm_N48_D32", "lstm", torch.bfloat16, B=3, T=9, N=48, D=32, seed=303, s0_var=1.0),
    fi.HeadwiseWorkload("bwd_elman_N40_D64", "elman", torch.bfloat16, B=5, T=9, N=40, D=64, seed=304, s0_var=1.0),
    fi.HeadwiseWorkload("bwd_lstm_B300_D64", "lstm", torch.bfloat16, B=300, T=5, N=1, D=64, seed=305, s0_var=1.0),
    fi.HeadwiseWorkload("bwd_gru_B130_N2_D256", "gru", torch.bfloat16, B=130, T=5, N=2, D=256, seed=306,
                        s0_var=1.0),
]
# fp32 heads wider than 64 units have no fused backward design (the single-workgroup fp32 design
# holds a head of at most 64 units; the die-local designs are bf16).
BWD_NO_FUSED_DESIGN = [
    fi.HeadwiseWorkload("bwd_lstm_f32_D128", "lstm", torch.float32, B=2, T=5, N=1, D=128, seed=307, s0_var=1.0),
    fi.HeadwiseWorkload("bwd_gru_f32_D256", "gru", torch.float32, B=3, T=4, N=2, D=256, seed=308, s0_var=1.0),
]


@pytest.mark.parametrize("w,path", [(w, p) for w in BWD_EXTREME for p in ("alternating", "fused")],
                         ids=lambda x: x if isinstance(x, str) else x.name)
def test_bwd_extreme_shapes(w, path):
    if path == "fused" and w.D == 1024:
        hw = _hw()
        plan = hw.frnn_bwd_plan_str(hw._desc(w.B, w.T, w.N, w.D, w.cell, w.dtype), "fused")
        assert "die-local-partials" in plan and ("KTL=2" if w.cell == "lstm" else "KTL=1") in plan, plan
    run_bwd_case(w, path)


def test_bwd_d1024_lds_design_full_launch():
    """Heads of 1024 units on the partial-sum design that keeps part of R in LDS (LSTM: two of a
    wave's four k-tiles; GRU: one of three), at 16 batch rows (8 groups of 2 rows, one per die, the
    whole chip) over 48 steps, against the oracle."""
    for cell, seed, ktl in (("lstm", 333, 2), ("gru", 334, 1)):
        w = fi.HeadwiseWorkload(f"bwd_{cell}_D1024_B16", cell, torch.bfloat16, B=16, T=48, N=1, D=1024, seed=seed,
                                s0_var=1.0)
        hw = _hw()
        plan = hw.frnn_bwd_plan_str(hw._desc(w.B, w.T, w.N, w.D, w.cell, w.dtype), "fused")
        assert f"KTL={ktl} " in plan and "groups=8 " in plan and "W=32 " in plan, plan
        run_bwd_case(w, "fused")


def test_bwd_d1024_lds_design_chunks():
    """Heads of 1024 units, 40 batch rows: two launches of 20 rows (7 groups of 3 rows) on the
    designs with R partly in LDS, LSTM and GRU, against the oracle."""
    for cell, seed in (("lstm", 335), ("gru", 336)):
        w = fi.HeadwiseWorkload(f"bwd_{cell}_D1024_B40", cell, torch.bfloat16, B=40, T=5, N=1, D=1024, seed=seed,
                                s0_var=1.0)
        hw = _hw()
        plan = hw.frnn_bwd_plan_str(hw._desc(w.B, w.T, w.N, w.D, w.cell, w.dtype), "fused")
        assert "KTL=" in plan and "chunks=2 " in plan, plan
        run_bwd_case(w, "fused")


def test_bwd_alternating_no_fused_design():
    """The heads the fused backward rejects run on the alternating path, against the oracle."""
    for w in BWD_NO_FUSED_DESIGN:
        run_bwd_case(w, "alternating")


@pytest.mark.parametrize("w", BWD_NO_FUSED_DESIGN, ids=lambda w: w.name)
def test_fused_bwd_rejects_heads_without_a_design(w):
    """The fused backward reports FRNN_EUNSUPPORTED for a head it has no design for, from the
    planner and from the compute call."""
    hw = _hw()
    desc = hw._desc(w.B, w.T, w.N, w.D, w.cell, w.dtype)
    with pytest.raises(hw.FrnnError) as ei:
        hw.frnn_bwd_plan_str(desc, "fused")
    assert ei.value.status == -2
    x = {k: (v.cuda() if v is not None else None) for k, v in fi.make_inputs(w).items()}
    ct = {k: (v.cuda() if v is not None else None) for k, v in fi.backward_cotangents(w).items()}
    st, _ = hw.frnn_fwd(x["Wx"], x["R"], x["b"], x["states0"], cell=w.cell, path="alternating")
    with pytest.raises(hw.FrnnError) as ei:
        hw.frnn_bwd(x["Wx"], x["R"], x["b"], x["states0"], st, ct["dstates"], ct["dlast"], cell=w.cell, path="fused")
    assert ei.value.status == -2


@pytest.mark.timeout(300)
@pytest.mark.parametrize("cell", ["lstm", "gru", "elman"])
def test_bwd_long_sequence_past_tag_wrap(cell):
    """65,600 steps: the fused backward's 16-bit step tags wrap (every step checked)."""
    w = fi.HeadwiseWorkload(f"bwd_{cell}_long", cell, torch.bfloat16, B=3, T=65600, N=1, D=64, seed=272, s0_var=1.0)
    env = {"FRNN_FUSED_BWD_PX": 1}  # a die-local design (an Elman head of 64 units takes the single workgroup)
    with _env(env):
        plan = _fused_plan_or_skip(w)
    assert "die-local" in plan, plan
    run_bwd_case(w, "fused", env=env)


_CH_GRU = fi.HeadwiseWorkload("bwd_gru_chunks_B40", "gru", torch.bfloat16, B=40, T=8, N=1, D=768, seed=251, s0_var=1.0)
_CH_LSTM = fi.HeadwiseWorkload("bwd_lstm_chunks_B40", "lstm", torch.bfloat16, B=40, T=6, N=1, D=768, seed=252,
                               s0_var=1.0)
_CH_ELMAN = fi.HeadwiseWorkload("bwd_elman_chunks_B64_N12", "elman", torch.bfloat16, B=64, T=16, N=12, D=64, seed=253,
                                s0_var=1.0)
# the single-workgroup design takes four 64-unit rows a workgroup: 128 rows of twelve heads need two
# launches of at most 21 groups of rows a head
_CH_ELMAN_L = fi.HeadwiseWorkload("bwd_elman_chunks_B128_N12", "elman", torch.bfloat16, B=128, T=16, N=12, D=64,
                                  seed=254, s0_var=1.0)


@pytest.mark.parametrize("w,px,chunks", [
    (_CH_GRU, 0, 3), (_CH_LSTM, 0, 3), (_CH_ELMAN, 0, 2),
    (_CH_GRU, 1, 2), (_CH_LSTM, 1, 2), (_CH_ELMAN, 1, 4), (_CH_ELMAN_L, 2, 2),
], ids=lambda x: getattr(x, "name", str(x)))
def test_bwd_fused_chunks(w, px, chunks):
    """A batch whose groups exceed one launch runs the fused serial part in chunks of rows (every
    design)."""
    with _env({"FRNN_FUSED_BWD_PX": px}):
        plan = _fused_plan_or_skip(w)
    assert f"chunks={chunks} " in plan and _DESIGN_NAME[px] in plan + " ", plan
    run_bwd_case(w, "fused", env={"FRNN_FUSED_BWD_PX": px})


_ELMAN_IN = fi.HeadwiseWorkload("bwd_elman_inputs_D64", "elman", torch.bfloat16, B=9, T=11, N=3, D=64, seed=214,
                                s0_var=1.0)


@pytest.mark.parametrize("raw", [1, 0])
@pytest.mark.parametrize("given", ["both", "dstates", "dlast", "no_states0"])
def test_bwd_elman_local_inputs(raw, given):
    """The single-workgroup design on an Elman cell: its I/O wave loads h and ds_h themselves (raw;
    no h.R recompute, the dR GEMM's h^T straight from the states) or two-float records
    (FRNN_BWD_ELMAN_RAW=0); either gradient of the forward's outputs may be absent (read as zeros),
    dlast joins ds_h only at the last time step, and an absent initial state reads as zeros."""
    hw = _hw()
    w = _ELMAN_IN
    assert "workgroup-local" in hw.frnn_bwd_plan_str(hw._desc(w.B, w.T, w.N, w.D, w.cell, w.dtype), "fused")
    x = {k: (v.cuda() if v is not None else None) for k, v in fi.make_inputs(w).items()}
    ct = fi.backward_cotangents(w)
    ds = ct["dstates"] if given != "dlast" else None
    dl = ct["dlast"] if given != "dstates" else None
    if given == "no_states0":
        x["states0"] = None
    _log(f"bwd case {w.name} raw={raw} given={given}")
    st, _ = hw.frnn_fwd(x["Wx"], x["R"], x["b"], x["states0"], cell="elman")
    with _env({"FRNN_BWD_ELMAN_RAW": raw}):
        grads = hw.frnn_bwd(x["Wx"], x["R"], x["b"], x["states0"], st, None if ds is None else ds.cuda(),
                            None if dl is None else dl.cuda(), cell="elman", path="fused")
    torch.cuda.synchronize()
    f = fi.to_f64
    ref = oracle.headwise_bwd("elman", f(x["Wx"]), f(x["R"]), f(x["b"]), f(x["states0"]), f(ds), f(dl))
    for name, gv, rv in zip(("dWx", "dR", "db", "dstates0"), grads, ref):
        e = float(np.abs(gv.double().cpu().numpy() - rv).max())
        scale = max(1.0, float(np.abs(rv).max()))
        assert e <= TOL[w.dtype] * scale, f"{name}: {e} > {TOL[w.dtype]} * {scale}"


def test_bwd_fused_matches_alternating():
    """The two backward paths agree closely (same operand roundings, different summation orders)."""
    hw = _hw()
    w = fi.HeadwiseWorkload("bwd_agree", "lstm", torch.bfloat16, B=8, T=40, N=2, D=256, seed=231, s0_var=1.0)
    x = {k: (v.cuda() if v is not None else None) for k, v in fi.make_inputs(w).items()}
    ct = {k: v.cuda() for k, v in fi.backward_cotangents(w).items()}
    st, _ = hw.frnn_fwd(x["Wx"], x["R"], x["b"], x["states0"], cell="lstm")
    ga = hw.frnn_bwd(x["Wx"], x["R"], x["b"], x["states0"], st, ct["dstates"], ct["dlast"], cell="lstm", path="alternating")
    gf = hw.frnn_bwd(x["Wx"], x["R"], x["b"], x["states0"], st, ct["dstates"], ct["dlast"], cell="lstm", path="fused")
    for a, f in zip(ga, gf):
        scale = max(1.0, a.abs().max().item())
        assert (a - f).abs().max().item() <= 1e-2 * scale


def test_bwd_t0():
    hw = _hw()
    dev = torch.device("cuda:0")
    for cell, G, S in (("lstm", 4, 2), ("gru", 3, 1)):
        Wx = torch.zeros((3, 0, G, 2, 64), dtype=torch.bfloat16, device=dev)
        R = torch.randn((G, 2, 64, 64), device=dev).to(torch.bfloat16)
        st = torch.zeros((S, 3, 0, 2, 64), device=dev)
        dlast = torch.randn((S, 3, 1, 2, 64), device=dev)
        dWx, dR, db, ds0 = hw.frnn_bwd(Wx, R, None, None, st, None, dlast, cell=cell)
        assert dWx.shape == (3, 0, G, 2, 64)
        assert torch.count_nonzero(dR).item() == 0 and torch.count_nonzero(db).item() == 0
        torch.testing.assert_close(ds0, dlast, rtol=0, atol=0)


def test_autograd_function_matches_frnn_bwd():
    """flashrnn() under torch autograd gives the gradients frnn_bwd returns (cast to the inputs'
    dtypes)."""
    hw = _hw()
    w = fi.HeadwiseWorkload("ag", "lstm", torch.float32, B=4, T=9, N=2, D=64, seed=221, s0_var=1.0)
    x = fi.make_inputs(w)
    ct = fi.backward_cotangents(w)
    dev = torch.device("cuda:0")
    leaves = [x[k].to(dev).requires_grad_(True) for k in ("Wx", "R", "b", "states0")]
    st, last = hw.flashrnn(*leaves, cell="lstm")
    loss = (st * ct["dstates"].to(dev)).sum() + (last * ct["dlast"].to(dev)).sum()
    loss.backward()
    ref = hw.frnn_bwd(*[t.detach() for t in leaves], st.detach(), ct["dstates"].to(dev), ct["dlast"].to(dev), cell="lstm")
    for leaf, r in zip(leaves, ref):
        torch.testing.assert_close(leaf.grad, r, rtol=1e-5, atol=1e-5)


# ------------------------------------------------------------------ multi-layer LSTM backward
def _stack_bwd_case(w, path):
    hw = _hw()
    x = fi.make_inputs(w)
    ct = fi.stack_cotangents(w)
    dev = torch.device("cuda:0")
    g = lambda t: None if t is None else t.to(dev)
    _log(f"stack bwd case {w.name} L={w.L} dirs={w.dirs} T={w.T} B={w.B} I={w.I} H={w.H} path={path}")
    got = hw.frnn_lstm_stack_bwd(g(x["x"]), [g(t) for t in x["Wi"]], [g(t) for t in x["Wh"]],
                                 [g(t) for t in x["b_ih"]], [g(t) for t in x["b_hh"]], g(x["h0"]), g(x["c0"]),
                                 g(ct["dout"]), g(ct["dhn"]), g(ct["dcn"]), path=path, bidirectional=w.dirs == 2)
    torch.cuda.synchronize()
    f = fi.to_f64
    ref = oracle.default().lstm_stack_bwd(f(x["x"]), [f(t) for t in x["Wi"]], [f(t) for t in x["Wh"]],
                                          [f(t) for t in x["b_ih"]], [f(t) for t in x["b_hh"]], f(x["h0"]),
                                          f(x["c0"]), f(ct["dout"]), f(ct["dhn"]), f(ct["dcn"]), dirs=w.dirs)
    names = ("dx", "dWi", "dWh", "db_ih", "db_hh", "dh0", "dc0")
    worst = 0.0
    for name, gv, rv in zip(names, got, ref):
        gl = gv if isinstance(gv, list) else [gv]
        rl = rv if isinstance(rv, list) else [rv]
        for k, (a, r) in enumerate(zip(gl, rl)):
            a = a.double().cpu().numpy()
            assert a.shape == r.shape and np.all(np.isfinite(a)), name
            scale = max(1.0, float(np.abs(r).max()))
            rel = float(np.abs(a - r).max()) / scale
            worst = max(worst, rel)
            assert rel <= TOL[torch.bfloat16], f"{name}[{k}]: max abs err / scale {rel}"
    _log(f"  worst max|err| / scale = {worst:.3e}")


STACK_BWD_SMALL = fi.StackWorkload("stack_bwd_small", torch.bfloat16, L=2, T=19, B=10, I=96, H=128, seed=261,
                                   zero_init=False)


@pytest.mark.parametrize("path", ["alternating", "fused"])
def test_stack_bwd_small(path):
    _stack_bwd_case(STACK_BWD_SMALL, path)


@pytest.mark.timeout(600)
def test_stack_bwd_full():
    # the float64 oracle takes about a minute at this size (every gradient depends on every step)
    _stack_bwd_case(fi.WORKLOADS["lstm2_bf16_T512_B32_I512_H512"], "fused")


# Two directions per layer (reading A21): direction 1 runs the backward through views that go from
# the last step to the first, and each layer's dX sums both directions'.
STACK_BWD_BIDIR = fi.StackWorkload("stack_bwd_bidir", torch.bfloat16, L=2, T=17, B=6, I=64, H=96, seed=262,
                                   zero_init=False, dirs=2)


@pytest.mark.parametrize("path", ["alternating", "fused"])
def test_stack_bwd_bidirectional(path):
    _stack_bwd_case(STACK_BWD_BIDIR, path)


@pytest.mark.timeout(900)
def test_stack_bwd_bidirectional_full():
    # the float64 oracle runs each direction of each layer forward and backward: about two minutes
    _stack_bwd_case(fi.get_workload("lstm2bi_bf16_T512_B32_I512_H512"), "fused")


@pytest.mark.parametrize("cell", ["lstm", "gru"])
@pytest.mark.parametrize("path", ["alternating", "fused"])
def test_bwd_negative_strides_time_reversed(path, cell):
    """frnn_bwd through the C ABI over views that run backwards in time (negative step strides,
    the pointers at step 0 of each view, which is the stored sequence's last step): Wx, the states,
    their gradients and dWx. Equals the oracle's backward of the time-order sequence."""
    hw = _hw()
    B, T, N, D = 5, 11, 2, 64
    G, S = {"lstm": (4, 2), "gru": (3, 1)}[cell]
    w = fi.HeadwiseWorkload(f"bwd_negstride_{cell}", cell, torch.bfloat16, B=B, T=T, N=N, D=D, seed=243, s0_var=1.0)
    x = fi.make_inputs(w)
    ct = fi.backward_cotangents(w)
    dev = torch.device("cuda:0")
    Wx, R, b, s0 = x["Wx"].to(dev), x["R"].to(dev), x["b"].to(dev), x["states0"].to(dev)
    st, _ = hw.frnn_fwd(Wx, R, b, s0, cell=cell, path="fused")           # time order
    wx_rev = Wx.flip(1).contiguous()                                     # stored last step first
    st_rev = st.flip(2).contiguous()
    ds_rev = ct["dstates"].to(dev).flip(2).contiguous()
    dl = ct["dlast"].to(dev).contiguous()
    dwx_rev = torch.full((B, T, G, N, D), float("nan"), dtype=torch.float32, device=dev)
    dR = torch.empty((G, N, D, D), dtype=torch.float32, device=dev)
    db = torch.empty((G, N, D), dtype=torch.float32, device=dev)
    ds0 = torch.empty((S, B, 1, N, D), dtype=torch.float32, device=dev)
    d = hw._desc(B, T, N, D, cell, torch.bfloat16)
    d.wx_sb, d.wx_st = T * G * N * D, -G * N * D
    d.st_ss, d.st_sb, d.st_st = B * T * N * D, T * N * D, -N * D
    wx0 = wx_rev.data_ptr() + (T - 1) * G * N * D * 2                    # element [0, 0] of each reversed view
    st0 = st_rev.data_ptr() + (T - 1) * N * D * 4
    ds0p = ds_rev.data_ptr() + (T - 1) * N * D * 4
    dwx0 = dwx_rev.data_ptr() + (T - 1) * G * N * D * 4
    ws = torch.empty(hw.frnn_bwd_workspace_bytes(d, path), dtype=torch.uint8, device=dev)
    hw.frnn_init()
    p = ctypes.c_void_p
    _log(f"bwd negative strides case cell={cell} path={path}")
    rc = hw.load().frnn_bwd(ctypes.byref(d), hw._path(path), p(wx0), p(R.data_ptr()), p(b.data_ptr()), p(s0.data_ptr()),
                            p(st0), p(ds0p), p(dl.data_ptr()), p(dwx0), p(dR.data_ptr()), p(db.data_ptr()),
                            p(ds0.data_ptr()), p(ws.data_ptr()), ws.numel(), hw._stream_handle(dev))
    assert rc == 0, hw.frnn_status_str(rc)
    hw.frnn_check(ws)
    f = fi.to_f64
    ref = oracle.headwise_bwd(cell, f(x["Wx"]), f(x["R"]), f(x["b"]), f(x["states0"]), f(ct["dstates"]), f(ct["dlast"]))
    got = (dwx_rev.flip(1), dR, db, ds0)
    for name, gv, rv in zip(("dWx", "dR", "db", "dstates0"), got, ref):
        gv = gv.double().cpu().numpy()
        scale = max(1.0, float(np.abs(rv).max()))
        err = float(np.abs(gv - rv).max())
        _log(f"  {name}: err={err:.3e} scale={scale:.3g}")
        assert np.all(np.isfinite(gv)) and err <= TOL[torch.bfloat16] * scale, name


@pytest.mark.parametrize("path", ["alternating", "fused"])
def test_bwd_strided_views(path):
    """frnn_bwd on a time-major Wx view, the recurrent weight Wh [D, 4D] read in place as R, and
    time-major states: dWx comes back with Wx's strides and dR with R's, equal to the oracle's
    gradients of the same values laid out densely."""
    hw = _hw()
    B, T, D = 6, 13, 128
    w = fi.HeadwiseWorkload("bwd_strided", "lstm", torch.bfloat16, B=B, T=T, N=1, D=D, seed=241, s0_var=1.0)
    x = fi.make_inputs(w)
    ct = fi.backward_cotangents(w)
    dev = torch.device("cuda:0")
    Wx_view = x["Wx"].permute(1, 0, 2, 3, 4).contiguous().to(dev).permute(1, 0, 2, 3, 4)
    Wh = x["R"][:, 0].permute(1, 0, 2).reshape(D, 4 * D).contiguous().to(dev)
    R_view = Wh.view(D, 4, D).permute(1, 0, 2).unsqueeze(1)
    st_tm = torch.empty((2, T, B, 1, D), dtype=torch.float32, device=dev)
    last = torch.empty((2, B, 1, 1, D), dtype=torch.float32, device=dev)
    b, s0 = x["b"].to(dev), x["states0"].to(dev)
    _log(f"bwd strided case path={path}")
    st_view = st_tm.permute(0, 2, 1, 3, 4)
    hw.frnn_fwd(Wx_view, R_view, b, s0, cell="lstm", path="fused", out=(st_view, last))
    grads = hw.frnn_bwd(Wx_view, R_view, b, s0, st_view, ct["dstates"].to(dev), ct["dlast"].to(dev), cell="lstm",
                        path=path)
    assert grads[0].stride() == Wx_view.stride() and grads[1].stride() == R_view.stride()
    f = fi.to_f64
    ref = oracle.headwise_bwd("lstm", f(x["Wx"]), f(x["R"]), f(x["b"]), f(x["states0"]), f(ct["dstates"]),
                              f(ct["dlast"]))
    for name, gv, rv in zip(("dWx", "dR", "db", "dstates0"), grads, ref):
        gv = gv.double().cpu().numpy()
        scale = max(1.0, float(np.abs(rv).max()))
        rel = float(np.abs(gv - rv).max()) / scale
        _log(f"  {name}: rel={rel:.2e}")
        assert rel <= TOL[torch.bfloat16], name
