"""HIP path against the fp64 oracle, element by element, on identical seeded inputs.

Tolerances (max abs error on h and c): 1e-4 for fp32 inputs, 3e-2 for bf16 inputs with fp32
accumulation. Every case, the full-size workloads in the launch configuration the benchmark times
included, compares every (batch, head) row element by element.
"""
import ctypes
import math
import os
import sys

import numpy as np
import pytest
import torch

import frnn_inputs as fi
import oracle

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 3e-2}


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


def run_case(w, path, pairs=None, env=None):
    hw = _hw()
    x = fi.make_inputs(w)
    dev = torch.device("cuda:0")
    args = {k: (v.to(dev) if v is not None else None) for k, v in x.items()}
    old = {}
    for k, v in (env or {}).items():
        old[k] = os.environ.get(k)
        os.environ[k] = str(v)
    try:
        _log(f"case {w.name} cell={w.cell} B={w.B} T={w.T} N={w.N} D={w.D} path={path} env={env}")
        st, last = hw.frnn_fwd(args["Wx"], args["R"], args["b"], args["states0"], cell=w.cell, path=path)
        torch.cuda.synchronize()
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    ref_st, ref_last = oracle.headwise_fwd(w.cell, fi.to_f64(x["Wx"]), fi.to_f64(x["R"]), fi.to_f64(x["b"]),
                                           fi.to_f64(x["states0"]), pairs=pairs)
    got = st.double().cpu().numpy()
    gl = last.double().cpu().numpy()
    if pairs is not None:
        bs = [p // w.N for p in pairs]
        ns = [p % w.N for p in pairs]
        got_s = np.stack([got[:, b, :, n] for b, n in zip(bs, ns)])
        ref_s = np.stack([ref_st[:, b, :, n] for b, n in zip(bs, ns)])
        gl_s = np.stack([gl[:, b, :, n] for b, n in zip(bs, ns)])
        rl_s = np.stack([ref_last[:, b, :, n] for b, n in zip(bs, ns)])
    else:
        got_s, ref_s, gl_s, rl_s = got, ref_st, gl, ref_last
    assert np.all(np.isfinite(got_s))
    err = np.abs(got_s - ref_s).max() if got_s.size else 0.0
    err_last = np.abs(gl_s - rl_s).max()
    sax = 0 if pairs is None else 1  # the state axis (h, c)
    err_h = np.abs(np.take(got_s, 0, sax) - np.take(ref_s, 0, sax)).max() if got_s.size else 0.0
    err_c = np.abs(np.take(got_s, 1, sax) - np.take(ref_s, 1, sax)).max() if got_s.size and w.S == 2 else 0.0
    _log(f"  max|err| states={err:.3e} (h {err_h:.3e}, c {err_c:.3e}) last={err_last:.3e}")
    tol = TOL[w.dtype]
    assert err <= tol, f"states max abs err {err} > {tol}"
    assert err_last <= tol
    # last_states is the final slice of states
    if w.T > 0:
        np.testing.assert_array_equal(gl, got[:, :, -1:])
    return err


SMALL = [
    fi.HeadwiseWorkload("lstm_bf16_ragged_D64", "lstm", torch.bfloat16, B=5, T=13, N=2, D=64, seed=101, s0_var=1.0),
    fi.HeadwiseWorkload("lstm_bf16_ragged_D96", "lstm", torch.bfloat16, B=19, T=7, N=2, D=96, seed=102, s0_var=0.5),
    fi.HeadwiseWorkload("lstm_bf16_D256", "lstm", torch.bfloat16, B=9, T=12, N=2, D=256, seed=103, s0_var=1.0, b_var=1.0),
    fi.HeadwiseWorkload("lstm_bf16_D512", "lstm", torch.bfloat16, B=6, T=6, N=1, D=512, seed=104),
    fi.HeadwiseWorkload("lstm_bf16_D768", "lstm", torch.bfloat16, B=16, T=5, N=1, D=768, seed=105),
    fi.HeadwiseWorkload("elman_bf16_ragged_D64", "elman", torch.bfloat16, B=21, T=9, N=3, D=64, seed=106, s0_var=1.0),
    fi.HeadwiseWorkload("elman_bf16_D128", "elman", torch.bfloat16, B=7, T=10, N=2, D=128, seed=107),
    fi.HeadwiseWorkload("elman_bf16_D512", "elman", torch.bfloat16, B=3, T=8, N=2, D=512, seed=108, s0_var=1.0),
    fi.HeadwiseWorkload("lstm_f32_D32", "lstm", torch.float32, B=3, T=11, N=2, D=32, seed=109, s0_var=1.0),
    fi.HeadwiseWorkload("lstm_f32_D64", "lstm", torch.float32, B=17, T=6, N=1, D=64, seed=110),
    fi.HeadwiseWorkload("elman_f32_D64", "elman", torch.float32, B=4, T=9, N=3, D=64, seed=111, s0_var=1.0),
    fi.HeadwiseWorkload("lstm_bf16_T1", "lstm", torch.bfloat16, B=1, T=1, N=1, D=64, seed=112, s0_var=1.0),
    fi.HeadwiseWorkload("gru_bf16_ragged_D64", "gru", torch.bfloat16, B=5, T=13, N=2, D=64, seed=113, s0_var=1.0),
    fi.HeadwiseWorkload("gru_bf16_ragged_D96", "gru", torch.bfloat16, B=19, T=7, N=2, D=96, seed=114, s0_var=0.5),
    fi.HeadwiseWorkload("gru_bf16_D256", "gru", torch.bfloat16, B=9, T=12, N=2, D=256, seed=115, s0_var=1.0, b_var=1.0),
    fi.HeadwiseWorkload("gru_bf16_D768", "gru", torch.bfloat16, B=16, T=5, N=1, D=768, seed=116),
    fi.HeadwiseWorkload("gru_f32_D32", "gru", torch.float32, B=3, T=11, N=2, D=32, seed=117, s0_var=1.0),
    fi.HeadwiseWorkload("gru_f32_D64", "gru", torch.float32, B=17, T=6, N=1, D=64, seed=118),
    fi.HeadwiseWorkload("gru_bf16_T1", "gru", torch.bfloat16, B=1, T=1, N=1, D=64, seed=119, s0_var=1.0),
]


@pytest.mark.parametrize("path", ["alternating", "fused"])
@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_small(w, path):
    if path == "fused" and w.dtype == torch.float32 and w.D > 64:
        pytest.skip("fp32 fused covers D <= 64")
    run_case(w, path)


# Die-local multi-workgroup design forced onto small shapes: several workgroups per group,
# several groups per die, ragged last batch block.
FORCED = [
    (fi.HeadwiseWorkload("lstm_forced_W4", "lstm", torch.bfloat16, B=7, T=9, N=3, D=64, seed=121, s0_var=1.0),
     {"FRNN_FUSED_W": 4, "FRNN_FUSED_BR": 3}),
    (fi.HeadwiseWorkload("lstm_forced_W8", "lstm", torch.bfloat16, B=11, T=6, N=2, D=128, seed=122, s0_var=1.0),
     {"FRNN_FUSED_W": 8, "FRNN_FUSED_BR": 4}),
    (fi.HeadwiseWorkload("elman_forced_W2", "elman", torch.bfloat16, B=9, T=8, N=2, D=64, seed=123, s0_var=1.0),
     {"FRNN_FUSED_W": 2, "FRNN_FUSED_BR": 4}),
    (fi.HeadwiseWorkload("lstm_forced_W16_BR4", "lstm", torch.bfloat16, B=15, T=5, N=1, D=256, seed=124),
     {"FRNN_FUSED_W": 16, "FRNN_FUSED_BR": 4}),
    (fi.HeadwiseWorkload("lstm_D768_8waves", "lstm", torch.bfloat16, B=16, T=9, N=1, D=768, seed=125, s0_var=1.0),
     {"FRNN_FUSED_NCW": 8}),
    (fi.HeadwiseWorkload("lstm_D768_4waves", "lstm", torch.bfloat16, B=16, T=9, N=1, D=768, seed=126, s0_var=1.0),
     {"FRNN_FUSED_NCW": 4}),
    (fi.HeadwiseWorkload("lstm_D512_W16_4waves", "lstm", torch.bfloat16, B=3, T=6, N=1, D=512, seed=127, s0_var=1.0),
     {"FRNN_FUSED_W": 16, "FRNN_FUSED_NCW": 4, "FRNN_FUSED_BR": 2}),
    (fi.HeadwiseWorkload("lstm_D512_W16_8waves", "lstm", torch.bfloat16, B=5, T=5, N=1, D=512, seed=128, s0_var=1.0),
     {"FRNN_FUSED_W": 16, "FRNN_FUSED_NCW": 8, "FRNN_FUSED_KS": 8, "FRNN_FUSED_BR": 2}),
    (fi.HeadwiseWorkload("lstm_D256_W16_8waves", "lstm", torch.bfloat16, B=5, T=7, N=2, D=256, seed=129, s0_var=1.0),
     {"FRNN_FUSED_W": 16, "FRNN_FUSED_NCW": 8, "FRNN_FUSED_BR": 2}),
    (fi.HeadwiseWorkload("gru_forced_W4", "gru", torch.bfloat16, B=7, T=9, N=3, D=64, seed=130, s0_var=1.0),
     {"FRNN_FUSED_W": 4, "FRNN_FUSED_BR": 3}),
    (fi.HeadwiseWorkload("gru_D768_8waves", "gru", torch.bfloat16, B=16, T=9, N=1, D=768, seed=132, s0_var=1.0),
     {"FRNN_FUSED_NCW": 8}),
    (fi.HeadwiseWorkload("gru_D768_6waves", "gru", torch.bfloat16, B=6, T=7, N=1, D=768, seed=133, s0_var=1.0),
     {"FRNN_FUSED_NCW": 6, "FRNN_FUSED_BR": 2}),
    (fi.HeadwiseWorkload("gru_D512_W16_4waves", "gru", torch.bfloat16, B=3, T=6, N=1, D=512, seed=134, s0_var=1.0),
     {"FRNN_FUSED_W": 16, "FRNN_FUSED_NCW": 4, "FRNN_FUSED_BR": 2}),
    # eight compute waves over a four-way K split (two waves per K range): four rows per group
    (fi.HeadwiseWorkload("lstm_D512_W16_8waves_KS4", "lstm", torch.bfloat16, B=7, T=6, N=2, D=512, seed=135,
                         s0_var=1.0), {"FRNN_FUSED_W": 16, "FRNN_FUSED_NCW": 8, "FRNN_FUSED_KS": 4, "FRNN_FUSED_BR": 4}),
    (fi.HeadwiseWorkload("gru_D512_W16_8waves_KS4", "gru", torch.bfloat16, B=5, T=6, N=1, D=512, seed=136,
                         s0_var=1.0), {"FRNN_FUSED_W": 16, "FRNN_FUSED_NCW": 8, "FRNN_FUSED_KS": 4, "FRNN_FUSED_BR": 4}),
]

# the design each forced case must get (compute waves, K split, tiles and k-tiles per wave)
FORCED_PLAN = {
    "lstm_D768_8waves": "NCW=8 KS=8 MTW=6 KTW=3",
    "lstm_D768_4waves": "NCW=4 KS=4 MTW=6 KTW=6",
    "lstm_D512_W16_4waves": "NCW=4 KS=4 MTW=8 KTW=4",
    "lstm_D512_W16_8waves": "NCW=8 KS=8 MTW=8 KTW=2",
    "lstm_D256_W16_8waves": "NCW=8 KS=8 MTW=4 KTW=1",
    "gru_D768_8waves": "NCW=8 KS=8 MTW=6 KTW=3",
    "gru_D768_6waves": "NCW=6 KS=6 MTW=6 KTW=4",
    "gru_D512_W16_4waves": "NCW=4 KS=4 MTW=8 KTW=4",
    "lstm_D512_W16_8waves_KS4": "NCW=8 KS=4 MTW=4 KTW=4",
    "gru_D512_W16_8waves_KS4": "NCW=8 KS=4 MTW=4 KTW=4",
}


@pytest.mark.parametrize("w,env", FORCED, ids=lambda x: getattr(x, "name", ""))
def test_forced_die_local(w, env):
    hw = _hw()
    old = {k: os.environ.get(k) for k in env}
    os.environ.update({k: str(v) for k, v in env.items()})
    try:
        plan = hw.frnn_plan_str(hw._desc(w.B, w.T, w.N, w.D, w.cell, w.dtype), "fused")
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    assert "die-local" in plan, plan
    if w.name in FORCED_PLAN:
        assert FORCED_PLAN[w.name] in plan, plan
    run_case(w, "fused", env=env)


# A whole Elman head per workgroup with at most four batch rows and two tiles per wave: the gates
# run one unit per lane after a DPP move (the lane's four units spread over four lanes). Ragged
# last block (B=7 in blocks of 3), full blocks of 4, and an initial state.
NARROW = [
    (fi.HeadwiseWorkload("elman_narrow_D128_BR3", "elman", torch.bfloat16, B=7, T=9, N=2, D=128, seed=135, s0_var=1.0),
     {"FRNN_FUSED_W": 1, "FRNN_FUSED_BR": 3}),
    (fi.HeadwiseWorkload("elman_narrow_D128_BR4", "elman", torch.bfloat16, B=8, T=11, N=3, D=128, seed=136),
     {"FRNN_FUSED_W": 1, "FRNN_FUSED_BR": 4}),
    (fi.HeadwiseWorkload("elman_narrow_D128_BR1", "elman", torch.bfloat16, B=2, T=5, N=1, D=128, seed=137, s0_var=1.0),
     {"FRNN_FUSED_W": 1, "FRNN_FUSED_BR": 1}),
]


@pytest.mark.parametrize("w,env", NARROW, ids=lambda x: getattr(x, "name", ""))
def test_forced_narrow_elman(w, env):
    hw = _hw()
    old = {k: os.environ.get(k) for k in env}
    os.environ.update({k: str(v) for k, v in env.items()})
    try:
        plan = hw.frnn_plan_str(hw._desc(w.B, w.T, w.N, w.D, w.cell, w.dtype), "fused")
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    assert "workgroup-local" in plan and f"BR={env['FRNN_FUSED_BR']} " in plan and "MTW=2 KTW=4" in plan, plan
    run_case(w, "fused", env=env)


@pytest.mark.parametrize("cell", ["lstm", "gru"])
def test_fused_batch_chunks(cell):
    """A batch that does not fit co-resident runs as several launches over chunks of rows: the
    chunk boundaries are invisible in the result."""
    hw = _hw()
    w = fi.HeadwiseWorkload(f"{cell}_chunks_B40", cell, torch.bfloat16, B=40, T=6, N=1, D=768, seed=241, s0_var=1.0)
    plan = hw.frnn_plan_str(hw._desc(w.B, w.T, w.N, w.D, w.cell, w.dtype), "fused")
    assert "chunks=3 " in plan, plan
    run_case(w, "fused")


@pytest.mark.parametrize("cell,G,S", [("lstm", 4, 2), ("gru", 3, 1)])
def test_t0_returns_initial_state(cell, G, S):
    hw = _hw()
    dev = torch.device("cuda:0")
    for path in ("alternating", "fused"):
        Wx = torch.zeros((3, 0, G, 2, 64), dtype=torch.bfloat16, device=dev)
        R = torch.randn((G, 2, 64, 64), device=dev).to(torch.bfloat16)
        s0 = torch.randn((S, 3, 1, 2, 64), device=dev).to(torch.bfloat16)
        st, last = hw.frnn_fwd(Wx, R, None, s0, cell=cell, path=path)
        assert st.shape == (S, 3, 0, 2, 64)
        torch.testing.assert_close(last, s0.float(), rtol=0, atol=0)
        st, last = hw.frnn_fwd(Wx, R, None, None, cell=cell, path=path)
        assert torch.count_nonzero(last).item() == 0


@pytest.mark.parametrize("cell", ["lstm", "gru"])
def test_continuation_matches_single_call(cell):
    hw = _hw()
    w = fi.HeadwiseWorkload("cont", cell, torch.bfloat16, B=6, T=20, N=2, D=128, seed=131, s0_var=1.0)
    x = {k: (v.cuda() if v is not None else None) for k, v in fi.make_inputs(w).items()}
    for path in ("alternating", "fused"):
        st, last = hw.frnn_fwd(x["Wx"], x["R"], x["b"], x["states0"], cell=cell, path=path)
        st1, last1 = hw.frnn_fwd(x["Wx"][:, :8].contiguous(), x["R"], x["b"], x["states0"], cell=cell, path=path)
        # the continuation starts from fp32 states rounded to the input dtype, so compare to tolerance
        st2, last2 = hw.frnn_fwd(x["Wx"][:, 8:].contiguous(), x["R"], x["b"], last1.to(torch.bfloat16), cell=cell,
                                 path=path)
        torch.testing.assert_close(st1, st[:, :, :8], rtol=0, atol=0)
        assert (st2 - st[:, :, 8:]).abs().max().item() < 3e-2


@pytest.mark.parametrize("cell", ["lstm", "gru"])
def test_fused_and_alternating_agree(cell):
    hw = _hw()
    w = fi.HeadwiseWorkload("agree", cell, torch.bfloat16, B=8, T=30, N=2, D=256, seed=141, s0_var=1.0)
    x = {k: (v.cuda() if v is not None else None) for k, v in fi.make_inputs(w).items()}
    a, _ = hw.frnn_fwd(x["Wx"], x["R"], x["b"], x["states0"], cell=cell, path="alternating")
    f, _ = hw.frnn_fwd(x["Wx"], x["R"], x["b"], x["states0"], cell=cell, path="fused")
    assert (a - f).abs().max().item() < 2e-2


# The exchange words carry a 16-bit step tag: a sequence longer than 65,536 steps wraps it. Die-local
# designs (the only ones that use tags) on a small head, every step checked against the oracle.
LONG_T = 65600


@pytest.mark.parametrize("cell,env", [("lstm", {"FRNN_FUSED_W": 4, "FRNN_FUSED_BR": 3}),
                                      ("gru", {"FRNN_FUSED_W": 4, "FRNN_FUSED_BR": 3}),
                                      ("elman", {"FRNN_FUSED_W": 2, "FRNN_FUSED_BR": 3})])
def test_long_sequence_past_tag_wrap(cell, env):
    w = fi.HeadwiseWorkload(f"{cell}_long_T{LONG_T}", cell, torch.bfloat16, B=3, T=LONG_T, N=1, D=64, seed=271,
                            s0_var=1.0)
    hw = _hw()
    old = {k: os.environ.get(k) for k in env}
    os.environ.update({k: str(v) for k, v in env.items()})
    try:
        plan = hw.frnn_plan_str(hw._desc(w.B, w.T, w.N, w.D, w.cell, w.dtype), "fused")
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    assert "die-local" in plan, plan
    run_case(w, "fused", env=env)


# Extreme shapes: the widest head the boundary takes (D = 1024; the LSTM and GRU heads' fused
# design keeps a quarter of R^T in LDS, since four gate rows of 1024 x 1024 bf16 are half of a
# die's register file), many narrow heads, and batches far past one launch's co-resident rows.
EXTREME = [
    fi.HeadwiseWorkload("lstm_D1024", "lstm", torch.bfloat16, B=2, T=6, N=1, D=1024, seed=291, s0_var=1.0),
    fi.HeadwiseWorkload("gru_D1024", "gru", torch.bfloat16, B=3, T=6, N=1, D=1024, seed=292, s0_var=1.0),
    fi.HeadwiseWorkload("elman_D1024", "elman", torch.bfloat16, B=3, T=7, N=1, D=1024, seed=293, s0_var=1.0),
    fi.HeadwiseWorkload("lstm_N48_D32", "lstm", torch.bfloat16, B=3, T=9, N=48, D=32, seed=294, s0_var=1.0),
    fi.HeadwiseWorkload("elman_N40_D64", "elman", torch.bfloat16, B=5, T=9, N=40, D=64, seed=295, s0_var=1.0),
    fi.HeadwiseWorkload("lstm_B300_D64", "lstm", torch.bfloat16, B=300, T=5, N=1, D=64, seed=296, s0_var=1.0),
    fi.HeadwiseWorkload("gru_B130_N2_D256", "gru", torch.bfloat16, B=130, T=5, N=2, D=256, seed=297, s0_var=1.0),
]


@pytest.mark.parametrize("path", ["alternating", "fused"])
@pytest.mark.parametrize("w", EXTREME, ids=lambda w: w.name)
def test_extreme_shapes(w, path):
    if path == "fused" and w.D == 1024 and w.cell != "elman":
        hw = _hw()
        assert "KTL=1" in hw.frnn_plan_str(hw._desc(w.B, w.T, w.N, w.D, w.cell, w.dtype), "fused")
    run_case(w, path)


def test_d1024_lds_design_full_launch():
    """Heads of 1024 units on the design that keeps a quarter of R^T in LDS, at 16 batch rows (8
    groups of 2 rows, one per die, the whole chip) over 64 steps, LSTM and GRU, against the oracle
    row by row."""
    for cell, seed in (("lstm", 331), ("gru", 332)):
        w = fi.HeadwiseWorkload(f"{cell}_D1024_B16", cell, torch.bfloat16, B=16, T=64, N=1, D=1024, seed=seed,
                                s0_var=1.0)
        hw = _hw()
        plan = hw.frnn_plan_str(hw._desc(w.B, w.T, w.N, w.D, w.cell, w.dtype), "fused")
        assert "KTL=1" in plan and "groups=8 " in plan, plan
        run_case(w, "fused")


# fp32 heads wider than 64 units have no fused design (the single-workgroup fp32 design holds a
# head of at most 64 units; the die-local designs are bf16).
NO_FUSED_DESIGN = [
    fi.HeadwiseWorkload("lstm_f32_D128", "lstm", torch.float32, B=2, T=5, N=1, D=128, seed=298, s0_var=1.0),
    fi.HeadwiseWorkload("gru_f32_D256", "gru", torch.float32, B=3, T=4, N=2, D=256, seed=299, s0_var=1.0),
]


@pytest.mark.parametrize("w", NO_FUSED_DESIGN, ids=lambda w: w.name)
def test_fused_rejects_heads_without_a_design(w):
    """The fused path reports FRNN_EUNSUPPORTED for a head it has no design for, from the planner
    and from the compute call, and leaves the outputs as they were."""
    hw = _hw()
    desc = hw._desc(w.B, w.T, w.N, w.D, w.cell, w.dtype)
    with pytest.raises(hw.FrnnError) as ei:
        hw.frnn_plan_str(desc, "fused")
    assert ei.value.status == -2
    x = {k: (v.cuda() if v is not None else None) for k, v in fi.make_inputs(w).items()}
    S = 2 if w.cell == "lstm" else 1
    out = (torch.full((S, w.B, w.T, w.N, w.D), 7.0, device="cuda"), torch.full((S, w.B, 1, w.N, w.D), 7.0, device="cuda"))
    with pytest.raises(hw.FrnnError) as ei:
        hw.frnn_fwd(x["Wx"], x["R"], x["b"], x["states0"], cell=w.cell, path="fused", out=out)
    assert ei.value.status == -2
    torch.cuda.synchronize()
    assert bool((out[0] == 7.0).all()) and bool((out[1] == 7.0).all())
    run_case(w, "alternating")  # the alternating path takes the shape


def test_repeat_calls_reuse_workspace():
    """Back-to-back calls on one workspace: the exchange buffer holds the previous call's tags."""
    hw = _hw()
    w = fi.HeadwiseWorkload("rep", "lstm", torch.bfloat16, B=16, T=17, N=1, D=256, seed=151)
    x = {k: (v.cuda() if v is not None else None) for k, v in fi.make_inputs(w).items()}
    d = hw._desc(16, 17, 1, 256, "lstm", torch.bfloat16)
    ws = torch.empty(hw.frnn_workspace_bytes(d, "fused"), dtype=torch.uint8, device="cuda")
    outs = [hw.frnn_fwd(x["Wx"], x["R"], x["b"], None, cell="lstm", path="fused", workspace=ws)[0] for _ in range(3)]
    for o in outs[1:]:
        torch.testing.assert_close(o, outs[0], rtol=0, atol=0)


# ------------------------------------------------------------------ full-size workloads
FULL_WORKLOADS = [
    "lstm_f32_B2_T16_N1_D32",
    "lstm_bf16_B8_T1024_N3_D256",
    "lstm_bf16_B16_T1024_N1_D768",
    "elman_bf16_B64_T2048_N12_D64",
    "gru_f32_B2_T16_N1_D32",
    "gru_bf16_B8_T1024_N3_D256",
    "gru_bf16_B16_T1024_N1_D768",
]


@pytest.mark.parametrize("path", ["fused", "alternating"])
@pytest.mark.parametrize("name", FULL_WORKLOADS)
def test_full_workload(name, path):
    # every (batch, head) row of the launch the benchmark times, element by element
    run_case(fi.get_workload(name), path)


def _stack_case(w, path, rows, env=None):
    if w.dirs > 1:
        return _stack_dirs_case(w, path, rows, env)

    hw = _hw()
    x = fi.make_inputs(w)
    dev = torch.device("cuda:0")
    _log(f"stack case {w.name} L={w.L} T={w.T} B={w.B} I={w.I} H={w.H} path={path} env={env}")
    g = lambda t: None if t is None else t.to(dev)
    old = {k: os.environ.get(k) for k in (env or {})}
    os.environ.update({k: str(v) for k, v in (env or {}).items()})
    try:
        out, hn, cn = hw.frnn_lstm_stack_fwd(g(x["x"]), [g(t) for t in x["Wi"]], [g(t) for t in x["Wh"]],
                                             [g(t) for t in x["b_ih"]], [g(t) for t in x["b_hh"]], g(x["h0"]),
                                             g(x["c0"]), path=path)
        torch.cuda.synchronize()
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    f = fi.to_f64
    sel = lambda a, axis: np.take(a, rows, axis=axis)
    ro, rh, rc = oracle.lstm_stack_p3(sel(f(x["x"]), 1), [f(t) for t in x["Wi"]], [f(t) for t in x["Wh"]],
                                      [f(t) for t in x["b_ih"]], [f(t) for t in x["b_hh"]],
                                      None if x["h0"] is None else sel(f(x["h0"]), 1),
                                      None if x["c0"] is None else sel(f(x["c0"]), 1))
    go = sel(out.double().cpu().numpy(), 1)
    gh = sel(hn.double().cpu().numpy(), 1)
    gc = sel(cn.double().cpu().numpy(), 1)
    e = max(np.abs(go - ro).max(), np.abs(gh - rh).max(), np.abs(gc - rc).max())
    _log(f"  max|err| out/hn/cn = {e:.3e}")
    assert np.isfinite(e) and e <= 3e-2


STACK_SMALL = fi.StackWorkload("stack_small", torch.bfloat16, L=2, T=19, B=10, I=96, H=128, seed=161, zero_init=False)


@pytest.mark.parametrize("path", ["fused", "alternating"])
def test_stack_small(path):
    _stack_case(STACK_SMALL, path, list(range(STACK_SMALL.B)))


def test_stack_small_register_staged_projection():
    # the first layer's bf16 projection through the register-staged GEMM instead of the LDS-DMA one
    _stack_case(STACK_SMALL, "fused", list(range(STACK_SMALL.B)), env={"FRNN_PROJ_DMA": 0})


@pytest.mark.parametrize("path", ["fused", "alternating"])
def test_stack_full(path):
    w = fi.WORKLOADS["lstm2_bf16_T512_B32_I512_H512"]
    _stack_case(w, path, list(range(w.B)))


def _stack_dirs_case(w, path, rows, env=None):
    """Multi-layer LSTM with two directions per layer against the oracle's layer-by-layer loops."""
    hw = _hw()
    x = fi.make_inputs(w)
    dev = torch.device("cuda:0")
    _log(f"bidirectional stack case {w.name} L={w.L} T={w.T} B={w.B} I={w.I} H={w.H} path={path} env={env}")
    g = lambda t: None if t is None else t.to(dev)
    old = {k: os.environ.get(k) for k in (env or {})}
    os.environ.update({k: str(v) for k, v in (env or {}).items()})
    try:
        out, hn, cn = hw.frnn_lstm_stack_fwd(g(x["x"]), [g(t) for t in x["Wi"]], [g(t) for t in x["Wh"]],
                                             [g(t) for t in x["b_ih"]], [g(t) for t in x["b_hh"]], g(x["h0"]),
                                             g(x["c0"]), path=path, bidirectional=True)
        torch.cuda.synchronize()
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    f = fi.to_f64
    sel = lambda a, axis: np.take(a, rows, axis=axis)
    ro, rh, rc = oracle.lstm_stack_dirs(sel(f(x["x"]), 1), [f(t) for t in x["Wi"]], [f(t) for t in x["Wh"]],
                                        [f(t) for t in x["b_ih"]], [f(t) for t in x["b_hh"]],
                                        None if x["h0"] is None else sel(f(x["h0"]), 1),
                                        None if x["c0"] is None else sel(f(x["c0"]), 1), dirs=2)
    go = sel(out.double().cpu().numpy(), 1)
    gh = sel(hn.double().cpu().numpy(), 1)
    gc = sel(cn.double().cpu().numpy(), 1)
    assert go.shape == ro.shape and gh.shape == rh.shape
    e = max(np.abs(go - ro).max(), np.abs(gh - rh).max(), np.abs(gc - rc).max())
    _log(f"  max|err| out/hn/cn = {e:.3e}")
    assert np.isfinite(e) and e <= 3e-2


STACK_BIDIR_SMALL = fi.StackWorkload("stack_bidir_small", torch.bfloat16, L=2, T=19, B=10, I=96, H=128, seed=162,
                                     zero_init=False, dirs=2)


@pytest.mark.parametrize("path", ["fused", "alternating"])
def test_stack_bidirectional_small(path):
    _stack_case(STACK_BIDIR_SMALL, path, list(range(STACK_BIDIR_SMALL.B)))


@pytest.mark.parametrize("path", ["fused", "alternating"])
def test_stack_bidirectional_three_layers(path):
    w = fi.StackWorkload("stack_bidir_l3", torch.bfloat16, L=3, T=7, B=5, I=64, H=64, seed=163, zero_init=False,
                         dirs=2)
    _stack_case(w, path, list(range(w.B)))


@pytest.mark.parametrize("path", ["fused", "alternating"])
def test_stack_bidirectional_full(path):
    w = fi.get_workload("lstm2bi_bf16_T512_B32_I512_H512")
    _stack_case(w, path, list(range(w.B)))


def test_stack_bidirectional_t0():
    hw = _hw()
    w = fi.StackWorkload("bidir_t0", torch.bfloat16, L=2, T=0, B=3, I=32, H=32, seed=164, zero_init=False, dirs=2)
    x = {k: v for k, v in fi.make_inputs(w).items()}
    g = lambda t: None if t is None else t.cuda()
    out, hn, cn = hw.frnn_lstm_stack_fwd(g(x["x"]), [g(t) for t in x["Wi"]], [g(t) for t in x["Wh"]],
                                         [g(t) for t in x["b_ih"]], [g(t) for t in x["b_hh"]], g(x["h0"]), g(x["c0"]),
                                         path="fused", bidirectional=True)
    torch.testing.assert_close(hn.cpu(), x["h0"].float(), rtol=0, atol=0)
    torch.testing.assert_close(cn.cpu(), x["c0"].float(), rtol=0, atol=0)


# ------------------------------------------------------------------ strided views (frnn_desc strides)
def test_strided_time_major_wx_and_wh_view():
    """A time-major projection [T,B,G*N*D] passed as Wx, the "5.3 LSTM" recurrent weight Wh [D,4D]
    read in place as R, and time-major states out, on both paths, against the oracle on the same
    values laid out densely."""
    hw = _hw()
    B, T, D = 6, 11, 128
    w = fi.HeadwiseWorkload("strided", "lstm", torch.bfloat16, B=B, T=T, N=1, D=D, seed=171, s0_var=1.0)
    x = fi.make_inputs(w)
    dev = torch.device("cuda:0")
    wx_tm = x["Wx"].permute(1, 0, 2, 3, 4).contiguous().to(dev)        # [T,B,G,1,D]
    Wx_view = wx_tm.permute(1, 0, 2, 3, 4)                            # [B,T,G,1,D], strides (G*D, B*G*D, ...)
    Wh = x["R"][:, 0].permute(1, 0, 2).reshape(D, 4 * D).contiguous().to(dev)   # Wh[d, g*D + e] = R[g,0,d,e]
    R_view = Wh.view(D, 4, D).permute(1, 0, 2).unsqueeze(1)           # [4,1,D,D], strides (D, *, 4D, 1)
    assert not Wx_view.is_contiguous() and not R_view.is_contiguous()
    ref, ref_last = oracle.headwise_fwd("lstm", fi.to_f64(x["Wx"]), fi.to_f64(x["R"]), fi.to_f64(x["b"]),
                                        fi.to_f64(x["states0"]))
    for path in ("fused", "alternating"):
        st_tm = torch.empty((2, T, B, 1, D), dtype=torch.float32, device=dev)
        last = torch.empty((2, B, 1, 1, D), dtype=torch.float32, device=dev)
        _log(f"strided case path={path}")
        hw.frnn_fwd(Wx_view, R_view, x["b"].to(dev), x["states0"].to(dev), cell="lstm", path=path,
                    out=(st_tm.permute(0, 2, 1, 3, 4), last))
        got = st_tm.permute(0, 2, 1, 3, 4).double().cpu().numpy()
        err = np.abs(got - ref).max()
        err_last = np.abs(last.double().cpu().numpy() - ref_last).max()
        _log(f"  max|err| states={err:.3e} last={err_last:.3e}")
        assert err <= 3e-2 and err_last <= 3e-2


def _desc_ptr_call(hw, d, path, Wx, R, b, s0, st, last):
    ws = torch.empty(hw.frnn_workspace_bytes(d, path), dtype=torch.uint8, device="cuda")
    hw.frnn_init()
    p = lambda t: None if t is None else ctypes.c_void_p(t)
    rc = hw.load().frnn_fwd(ctypes.byref(d), hw._path(path), p(Wx), p(R), p(b), p(s0), p(st), p(last),
                            ctypes.c_void_p(ws.data_ptr()), ws.numel(), hw._stream_handle(torch.device("cuda:0")))
    assert rc == 0, hw.frnn_status_str(rc)
    hw.frnn_check(ws)


@pytest.mark.parametrize("path", ["fused", "alternating"])
def test_negative_strides_time_reversed(path):
    """Negative strides through the C ABI: Wx read backwards in time (the pointer at step 0 of the
    view, which is the stored sequence's last step) and states written backwards, equal the
    forward over the reversed sequence."""
    hw = _hw()
    B, T, N, D = 5, 9, 2, 64
    w = fi.HeadwiseWorkload("negstride", "lstm", torch.bfloat16, B=B, T=T, N=N, D=D, seed=172, s0_var=1.0)
    x = fi.make_inputs(w)
    dev = torch.device("cuda:0")
    stored = x["Wx"].flip(1).contiguous().to(dev)                      # the sequence stored last step first
    R, b, s0 = x["R"].to(dev), x["b"].to(dev), x["states0"].to(dev)
    st = torch.full((2, B, T, N, D), float("nan"), dtype=torch.float32, device=dev)
    last = torch.empty((2, B, 1, N, D), dtype=torch.float32, device=dev)
    d = hw._desc(B, T, N, D, "lstm", torch.bfloat16)
    G = 4
    d.wx_sb, d.wx_st = T * G * N * D, -G * N * D
    d.st_ss, d.st_sb, d.st_st = B * T * N * D, T * N * D, -N * D
    wx0 = stored.data_ptr() + (T - 1) * G * N * D * 2                 # element [0, 0] of the reversed view
    st0 = st.data_ptr() + (T - 1) * N * D * 4
    _desc_ptr_call(hw, d, path, wx0, R.data_ptr(), b.data_ptr(), s0.data_ptr(), st0, last.data_ptr())
    got = st.flip(2).double().cpu().numpy()                            # written backwards: flip to time order
    ref, ref_last = oracle.headwise_fwd("lstm", fi.to_f64(x["Wx"]), fi.to_f64(x["R"]), fi.to_f64(x["b"]),
                                        fi.to_f64(x["states0"]))
    err = np.abs(got - ref).max()
    _log(f"  negative strides {path}: max|err| states={err:.3e}")
    assert np.all(np.isfinite(got)) and err <= 3e-2
    assert np.abs(last.double().cpu().numpy() - ref_last).max() <= 3e-2



def test_die_local_after_graph_replay():
    """A die-local launch right after a HIP graph replay: the replay changes how the hardware deals
    the next launch's workgroups to dies (workgroup i no longer lands on die i % 8), so groups are
    formed from the workgroups that really share a die. Forward and backward, every replay checked."""
    hw = _hw()
    dev = torch.device("cuda:0")
    w = fi.HeadwiseWorkload("after_graph", "lstm", torch.bfloat16, B=16, T=24, N=1, D=768, seed=184, s0_var=1.0)
    assert "die-local" in hw.frnn_plan_str(hw._desc(w.B, w.T, w.N, w.D, w.cell, w.dtype), "fused")
    x = {k: (v.to(dev) if v is not None else None) for k, v in fi.make_inputs(w).items()}
    ref, _ = oracle.headwise_fwd("lstm", *(fi.to_f64(v) for v in fi.make_inputs(w).values()))
    buf = torch.ones(1 << 16, device=dev)
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        buf.mul_(1.0)  # warm the kernel outside the capture
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            buf.mul_(1.0)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        graph.replay()
        st, last = hw.frnn_fwd(x["Wx"], x["R"], x["b"], x["states0"], cell="lstm", path="fused")  # checks the error word
        err = float(np.abs(st.double().cpu().numpy() - ref).max())
        _log(f"  replay {rep}: forward max|err| = {err:.3e}")
        assert err <= 3e-2
        graph.replay()
        ct = {k: v.to(dev) for k, v in fi.backward_cotangents(w).items()}
        hw.frnn_bwd(x["Wx"], x["R"], x["b"], x["states0"], st, ct["dstates"], ct["dlast"], cell="lstm", path="fused")
    assert float(buf[0]) == 1.0
