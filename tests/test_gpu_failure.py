"""Failure handling of the fused kernels' bounded waits, forced from the host.

Every inter-workgroup wait of the fused kernels is bounded by a wall-clock limit; when one runs
out, the workgroup records FRNN_ETIMEOUT in the workspace's error word, raises the abort flag that
every wave of it looks at after the step's barrier, and all its waves leave at that barrier; the
other workgroups see the error word in their own polls and leave the same way. These tests make
one step publish a stale tag (the FRNN_TEST_STALL_STEP hook, never set in a normal call), so that
its consumers' waits run out for real under a short limit (FRNN_TIMEOUT_MS), and check that the
call reports FRNN_ETIMEOUT through frnn_check and that the next call on the same workspace is
correct. Every kernel exits normally; nothing waits without a bound.
"""
import os

import numpy as np
import pytest
import torch

import frnn_inputs as fi
import oracle

pytestmark = pytest.mark.gpu

ETIMEOUT = -6


def _hw():
    import head_wise_lstm_amd as hw
    return hw


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    _hw().load()


class _env:
    def __init__(self, env):
        self.env = {k: str(v) for k, v in env.items()}

    def __enter__(self):
        self.old = {k: os.environ.get(k) for k in self.env}
        os.environ.update(self.env)

    def __exit__(self, *exc):
        for k, v in self.old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


STALL = {"FRNN_TEST_STALL_STEP": 5, "FRNN_TIMEOUT_MS": 50}


def _inputs(w):
    return {k: (v.cuda() if v is not None else None) for k, v in fi.make_inputs(w).items()}


@pytest.mark.parametrize("shape", [(16, 768, "lstm"), (8, 256, "gru"), (4, 512, "elman")])
def test_fwd_wait_runs_out_then_next_call_is_clean(shape):
    hw = _hw()
    B, D, cell = shape
    w = fi.HeadwiseWorkload(f"stall_{cell}", cell, torch.bfloat16, B=B, T=40, N=1, D=D, seed=181, s0_var=1.0)
    d = hw._desc(w.B, w.T, w.N, w.D, w.cell, w.dtype)
    plan = hw.frnn_plan_str(d, "fused")
    print(f"stall forward {w.name}: {plan}", flush=True)
    assert "die-local" in plan, plan  # the design whose workgroups wait on each other
    x = _inputs(w)
    ws = torch.empty(hw.frnn_workspace_bytes(d, "fused"), dtype=torch.uint8, device="cuda")
    with _env(STALL):
        hw.frnn_fwd(x["Wx"], x["R"], x["b"], x["states0"], cell=cell, path="fused", workspace=ws, check=False)
    with pytest.raises(hw.FrnnError) as e:
        hw.frnn_check(ws)
    assert e.value.status == ETIMEOUT
    # the same workspace, no hook: the call clears the error word and the exchange buffer
    st, last = hw.frnn_fwd(x["Wx"], x["R"], x["b"], x["states0"], cell=cell, path="fused", workspace=ws)
    ref, _ = oracle.headwise_fwd(cell, *(fi.to_f64(v) for v in fi.make_inputs(w).values()))
    err = float(np.abs(st.double().cpu().numpy() - ref).max())
    print(f"  after the timeout: max|err| = {err:.3e}", flush=True)
    assert err <= 3e-2


@pytest.mark.parametrize("px", [1, 0])
def test_bwd_wait_runs_out_then_next_call_is_clean(px):
    hw = _hw()
    w = fi.HeadwiseWorkload("stall_bwd", "lstm", torch.bfloat16, B=8, T=40, N=1, D=256, seed=182, s0_var=1.0)
    d = hw._desc(w.B, w.T, w.N, w.D, w.cell, w.dtype)
    with _env({"FRNN_FUSED_BWD_PX": px}):
        plan = hw.frnn_bwd_plan_str(d, "fused")
    print(f"stall backward: {plan}", flush=True)
    assert ("die-local-partials" in plan) == bool(px), plan
    x = _inputs(w)
    ct = {k: v.cuda() for k, v in fi.backward_cotangents(w).items()}
    st, _ = hw.frnn_fwd(x["Wx"], x["R"], x["b"], x["states0"], cell="lstm", path="fused")
    ws = torch.empty(hw.frnn_bwd_workspace_bytes(d, "fused"), dtype=torch.uint8, device="cuda")
    with _env(dict(STALL, FRNN_FUSED_BWD_PX=px)):
        hw.frnn_bwd(x["Wx"], x["R"], x["b"], x["states0"], st, ct["dstates"], ct["dlast"], cell="lstm", path="fused",
                    workspace=ws, check=False)
    with pytest.raises(hw.FrnnError) as e:
        hw.frnn_check(ws)
    assert e.value.status == ETIMEOUT
    with _env({"FRNN_FUSED_BWD_PX": px}):
        grads = hw.frnn_bwd(x["Wx"], x["R"], x["b"], x["states0"], st, ct["dstates"], ct["dlast"], cell="lstm",
                            path="fused", workspace=ws)
    f = fi.to_f64
    raw = fi.make_inputs(w)
    ref = oracle.headwise_bwd("lstm", f(raw["Wx"]), f(raw["R"]), f(raw["b"]), f(raw["states0"]),
                              f(ct["dstates"].cpu()), f(ct["dlast"].cpu()))
    for name, gv, rv in zip(("dWx", "dR", "db", "dstates0"), grads, ref):
        rel = float(np.abs(gv.double().cpu().numpy() - rv).max()) / max(1.0, float(np.abs(rv).max()))
        print(f"  after the timeout: {name} rel={rel:.2e}", flush=True)
        assert rel <= 1e-2, name
