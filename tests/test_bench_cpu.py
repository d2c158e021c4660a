"""Host logic of bench.py's measurement path, on synthetic rocprofv3 counter files (no GPU)."""
import csv
import json
import os
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
KERNEL = "void frnn::fused_fwd_kernel<0, false, false, 8, 8, 6, 3>(frnn::FusedArgs)"


def _write_counters(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, value) in enumerate(rows, start=1):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": "X", "Counter_Value": value})


def test_counter_mean_takes_the_last_dispatches_in_order(tmp_path):
    p = tmp_path / "c.csv"
    # input copies first (small), then the kernel, then five calibration copies
    _write_counters(p, [("__amd_rocclr_copyBuffer", 3.0), ("__amd_rocclr_copyBuffer", 5.0), (KERNEL, 100.0),
                        (KERNEL, 102.0)] + [("__amd_rocclr_copyBuffer", 1000.0 + i) for i in range(5)])
    mean, n, names = bench._counter_mean(str(p), "copyBuffer", last=5)
    assert n == 5 and mean == pytest.approx(1002.0) and names == ["__amd_rocclr_copyBuffer"]
    mean, n, _ = bench._counter_mean(str(p), "copyBuffer")
    assert n == 7 and mean == pytest.approx((3 + 5 + 5 * 1002.0) / 7)
    mean, n, names = bench._counter_mean(str(p), "fused_fwd_kernel")
    assert n == 2 and mean == pytest.approx(101.0) and names == [KERNEL]
    with pytest.raises(SystemExit):
        bench._counter_mean(str(p), "no_such_kernel")


def test_write_traffic_scales_by_the_copy_calibration(tmp_path):
    # a copy of 256 MiB that FETCH_SIZE reads as half its size and WRITE_SIZE as its size: factors 2 and 1
    true_kib = 256 * 1024.0
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _write_counters(fetch, [("__amd_rocclr_copyBuffer", 7.0), (KERNEL, 1000.0), (KERNEL, 1002.0)]
                    + [("__amd_rocclr_copyBuffer", true_kib / 2)] * 5)
    _write_counters(write, [("__amd_rocclr_copyBuffer", 9.0), (KERNEL, 500.0), (KERNEL, 500.0)]
                    + [("__amd_rocclr_copyBuffer", true_kib)] * 5)
    tj = tmp_path / "traffic.json"
    args = types.SimpleNamespace(write_traffic=[str(fetch), str(write), str(fetch), str(write)], backward=False,
                                 path="fused", copy_mib=256, workload="lstm_bf16_B16_T1024_N1_D768",
                                 traffic_json=str(tj))
    bench.write_traffic(args)
    e = json.load(open(tj))["lstm_bf16_B16_T1024_N1_D768:fused"]
    assert e["fetch_factor"] == pytest.approx(2.0) and e["write_factor"] == pytest.approx(1.0)
    assert e["read_bytes"] == pytest.approx(1001.0 * 1024 * 2) and e["write_bytes"] == pytest.approx(500.0 * 1024)
    assert e["bytes_per_launch"] == pytest.approx(e["read_bytes"] + e["write_bytes"])
    # algorithmic bytes of the headline: Wx, R, b read once (bf16), h and c written once (fp32)
    B, T, N, D, G = 16, 1024, 1, 768, 4
    alg = (B * T * G * N * D + G * N * D * D + G * N * D) * 2 + 2 * B * T * N * D * 4 + 2 * B * N * D * 4
    assert e["algorithmic_bytes"] == alg
    assert e["kernel_sources_sha256_16"] == bench.kernel_sources_hash()


def test_write_traffic_backward_algorithmic_bytes(tmp_path):
    # the partial-sum serial kernel's own bytes: 8-float step records read once, dWx (fp32) and the
    # dR operand da (bf16) of every gate written once, R read once
    kname = "void frnn::fused_bwdx_kernel<0, 8, 6, 3, 0>(frnn::FusedBwdArgs)"
    true_kib = 256 * 1024.0
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _write_counters(fetch, [(kname, 100.0)] + [("__amd_rocclr_copyBuffer", true_kib)] * 5)
    _write_counters(write, [(kname, 50.0)] + [("__amd_rocclr_copyBuffer", true_kib)] * 5)
    tj = tmp_path / "traffic.json"
    args = types.SimpleNamespace(write_traffic=[str(fetch), str(write), str(fetch), str(write)], backward=True,
                                 path="fused", copy_mib=256, workload="lstm_bf16_B16_T1024_N1_D768",
                                 traffic_json=str(tj))
    bench.write_traffic(args)
    e = json.load(open(tj))["lstm_bf16_B16_T1024_N1_D768:fused:backward"]
    B, T, N, D, G = 16, 1024, 1, 768, 4
    assert e["kernel"] == kname
    assert e["algorithmic_bytes"] == B * T * N * D * (8 * 4 + G * (4 + 2)) + G * N * D * D * 2 == 709361664


def test_headwise_flops_and_bytes():
    w = types.SimpleNamespace(B=16, T=1024, N=1, D=768, G=4, S=2, s0_var=None)
    assert bench.headwise_flops(w) == 2.0 * 16 * 1 * 4 * 768 * 768 * 1024 == pytest.approx(77.31e9, rel=1e-3)
    assert bench.headwise_bytes(w, 2) == pytest.approx(206149632.0)
