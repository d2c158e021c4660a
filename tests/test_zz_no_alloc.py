"""frnn_fwd_noalloc, the entry point for callers that cannot allocate device memory, against
frnn_fwd on the same inputs: two calls in a row, the second smaller, on both paths (the library's
array keeps the first call's contents; the second must not read them)."""
import ctypes

import numpy as np
import pytest
import torch

import frnn_inputs as fi

pytestmark = pytest.mark.gpu


def _hw():
    import head_wise_lstm_amd as hw
    return hw


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    _hw().load()


CASES = [
    fi.HeadwiseWorkload("noalloc_big", "lstm", torch.bfloat16, B=16, T=48, N=1, D=768, seed=191, s0_var=1.0),
    fi.HeadwiseWorkload("noalloc_small", "lstm", torch.bfloat16, B=5, T=13, N=2, D=128, seed=192, s0_var=1.0),
]


def _run(hw, w, path, noalloc):
    x = {k: (v.cuda() if v is not None else None) for k, v in fi.make_inputs(w).items()}
    out = (torch.full((w.S, w.B, w.T, w.N, w.D), float("nan"), device="cuda"),
           torch.full((w.S, w.B, 1, w.N, w.D), float("nan"), device="cuda"))
    if noalloc:
        # straight through the C ABI: descriptor, raw pointers, torch's stream
        d = hw._desc(w.B, w.T, w.N, w.D, w.cell, w.dtype)
        hw.frnn_init()
        p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
        st = hw._stream_handle(torch.device("cuda:0"))
        rc = hw.load().frnn_fwd_noalloc(ctypes.byref(d), hw._path(path), p(x["Wx"]), p(x["R"]), p(x["b"]),
                                        p(x["states0"]), p(out[0]), p(out[1]), st)
        assert rc == 0, hw.frnn_status_str(rc)
        assert hw.load().frnn_check(None, st) == 0
    else:
        hw.frnn_fwd(x["Wx"], x["R"], x["b"], x["states0"], cell=w.cell, path=path, out=out)
    torch.cuda.synchronize()
    return [t.cpu() for t in out]


@pytest.mark.parametrize("path", ["fused", "alternating"])
def test_noalloc_matches_frnn_fwd_twice(path):
    hw = _hw()
    for w in CASES:  # the second call is smaller than the first
        print(f"noalloc {w.name} B={w.B} T={w.T} N={w.N} D={w.D} path={path}", flush=True)
        got = _run(hw, w, path, True)
        ref = _run(hw, w, path, False)
        for g, r in zip(got, ref):
            assert torch.isfinite(g).all()
            err = float((g.double() - r.double()).abs().max())
            print(f"  max|noalloc - frnn_fwd| = {err:.3e}", flush=True)
            assert err <= 3e-2


def test_noalloc_binding_and_size_limit():
    hw = _hw()
    w = CASES[1]
    x = {k: (v.cuda() if v is not None else None) for k, v in fi.make_inputs(w).items()}
    out = (torch.empty((w.S, w.B, w.T, w.N, w.D), device="cuda"), torch.empty((w.S, w.B, 1, w.N, w.D), device="cuda"))
    st, last = hw.frnn_fwd_noalloc(x["Wx"], x["R"], x["b"], x["states0"], out, cell="lstm")
    ref, ref_last = hw.frnn_fwd(x["Wx"], x["R"], x["b"], x["states0"], cell="lstm")
    assert float((st - ref).abs().max()) <= 3e-2 and float((last - ref_last).abs().max()) <= 3e-2
    # a problem needing more than the array is refused before anything is enqueued
    big = hw._desc(64, 8, 4, 1024, "lstm", torch.bfloat16)
    assert hw.load().frnn_fwd_noalloc(ctypes.byref(big), 1, None, None, None, None, None, None, None) == -3
