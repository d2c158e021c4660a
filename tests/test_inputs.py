"""The seeded input generator: determinism and the stated distributions."""
import math

import numpy as np
import torch

import frnn_inputs as fi


def test_deterministic_and_distinct_seeds():
    w = fi.HeadwiseWorkload("t", "lstm", torch.bfloat16, B=3, T=7, N=2, D=32, seed=5, s0_var=1.0)
    a, b = fi.make_inputs(w), fi.make_inputs(w)
    for k in a:
        assert fi.sha256_of(a[k]) == fi.sha256_of(b[k])
    w2 = fi.HeadwiseWorkload("t", "lstm", torch.bfloat16, B=3, T=7, N=2, D=32, seed=6, s0_var=1.0)
    assert fi.sha256_of(fi.make_inputs(w2)["Wx"]) != fi.sha256_of(a["Wx"])


def test_headwise_shapes_dtypes_and_variances():
    w = fi.WORKLOADS["lstm_bf16_B8_T1024_N3_D256"]
    x = fi.make_inputs(w)
    assert x["Wx"].shape == (8, 1024, 4, 3, 256) and x["Wx"].dtype == torch.bfloat16
    assert x["R"].shape == (4, 3, 256, 256)
    assert x["b"].shape == (4, 3, 256)
    assert x["states0"].shape == (2, 8, 1, 3, 256)
    assert abs(x["Wx"].float().var().item() - 1.0) < 0.01
    assert abs(x["R"].float().var().item() - 1.0 / 256) < 1e-4
    assert abs(x["b"].float().var().item() - 1.0) < 0.05
    w3 = fi.WORKLOADS["lstm_bf16_B16_T1024_N1_D768"]
    assert w3.s0_var is None and fi.make_inputs(w3)["states0"] is None


def test_stack_inputs_uniform_bound():
    w = fi.WORKLOADS["lstm2_bf16_T512_B32_I512_H512"]
    x = fi.make_inputs(w)
    bound = 1.0 / math.sqrt(512)
    assert x["x"].shape == (512, 32, 512)
    for l in range(2):
        assert x["Wi"][l].shape == (512, 2048) and x["Wh"][l].shape == (512, 2048)
        assert x["b_ih"][l].shape == (2048,) and x["b_hh"][l].shape == (2048,)
        assert x["Wh"][l].float().abs().max().item() <= bound * 1.004
    assert x["h0"] is None and x["c0"] is None


def test_to_f64_exact():
    t = torch.tensor([1.0, -2.5, 3.140625], dtype=torch.bfloat16)
    np.testing.assert_array_equal(fi.to_f64(t), np.array([1.0, -2.5, 3.140625]))


def test_gru_workloads_shapes():
    for name, w in fi.GRU_WORKLOADS.items():
        assert fi.get_workload(name) is w and w.cell == "gru" and (w.G, w.S) == (3, 1)
    x = fi.make_inputs("gru_f32_B2_T16_N1_D32")
    assert tuple(x["Wx"].shape) == (2, 16, 3, 1, 32) and tuple(x["R"].shape) == (3, 1, 32, 32)
    assert tuple(x["b"].shape) == (3, 1, 32) and tuple(x["states0"].shape) == (1, 2, 1, 1, 32)


def test_bidirectional_stack_workload():
    w = fi.get_workload("lstm2bi_bf16_T512_B32_I512_H512")
    assert w.dirs == 2 and (w.L, w.T, w.B, w.I, w.H) == (2, 512, 32, 512, 512)
    x = fi.make_inputs(w)
    assert len(x["Wi"]) == len(x["Wh"]) == len(x["b_ih"]) == len(x["b_hh"]) == 4
    assert [tuple(t.shape) for t in x["Wi"]] == [(512, 2048), (512, 2048), (1024, 2048), (1024, 2048)]
    # one direction: the same draws as before the direction count existed
    one = fi.StackWorkload("one", torch.bfloat16, L=2, T=3, B=2, I=8, H=32, seed=9)
    a = fi.make_inputs(one)
    assert [tuple(t.shape) for t in a["Wi"]] == [(8, 128), (32, 128)]
