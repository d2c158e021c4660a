#!/usr/bin/env python3
"""Benchmark of the head-wise LSTM forward recurrence on one MI355X.

A step is one full forward call (all T timesteps of the recurrence) over one batch of synthetic
inputs already resident in device memory. Default workload: LSTM, bf16 inputs with fp32
accumulation, B=16, T=1024, N=1 head, D=768 (gates i, f, z, o), fused path.

Prints ONE JSON line: the metric (achieved TFLOP/s of the recurrent contraction, with
microseconds per timestep beside it), a roofline object for the dominant kernel measured with HIP
events on the stream the kernel runs on, and the fp64 oracle timed on a bounded sample on the
host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "LSTM fwd µs/timestep + achieved TFLOP/s (% MFMA bf16 peak), B=16 N=1 D=768"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, at the 2.4 GHz peak engine clock
PEAK_SCLK_MHZ = 2400.0
PEAK_HBM_GBS = 8000.0
WS_RING_BYTES = 24 << 30   # workspaces of the timed calls: each call its own where they fit (288 GB of HBM)


def headwise_flops(w) -> float:
    """Algorithmic FLOPs of one forward call: the recurrent contraction only, 2*B*N*G*D^2*T."""
    return 2.0 * w.B * w.N * w.G * w.D * w.D * w.T


def headwise_bytes(w, elt: int) -> float:
    """Algorithmic HBM bytes of one call: Wx, R, b, states0 read once; states written once (fp32)."""
    rd = (w.B * w.T * w.G * w.N * w.D + w.G * w.N * w.D * w.D + w.G * w.N * w.D) * elt
    if w.s0_var is not None:
        rd += w.S * w.B * w.N * w.D * elt
    wr = w.S * w.B * w.T * w.N * w.D * 4 + w.S * w.B * w.N * w.D * 4
    return float(rd + wr)


def kernel_sources_hash() -> str:
    """First 16 hex digits of sha256 over the HIP sources (any change to them stales a traffic figure)."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "head_wise_lstm_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def _counter_mean(csv_path: str, name_part: str, last: int = 0) -> tuple:
    """Mean Counter_Value (KiB per dispatch) over the dispatches of the kernels whose name holds
    name_part (only the last `last` of them, in dispatch order, when last > 0)."""
    import csv
    rows = []
    with open(csv_path, newline="") as f:
        for row in csv.DictReader(f):
            if name_part in row["Kernel_Name"]:
                rows.append(row)
    if last:
        rows = sorted(rows, key=lambda r: int(r.get("Dispatch_Id", 0)))[-last:]
    vals = [float(r["Counter_Value"]) for r in rows]
    names = {r["Kernel_Name"] for r in rows}
    if not vals:
        raise SystemExit(f"{csv_path}: no dispatch of a kernel named like {name_part!r}")
    return sum(vals) / len(vals), len(vals), sorted(names)


def write_traffic(args) -> None:
    """Turn four rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE and WRITE_SIZE of the
    benchmark, then of --copy-calibration) into a per-launch HBM byte figure in --traffic-json."""
    import frnn_inputs as fi
    fetch_csv, write_csv, fetch_copy_csv, write_copy_csv = args.write_traffic
    if args.backward:
        kname = "fused_bwd" if args.path == "fused" else "bwd_dh_kernel"  # either fused backward design
    else:
        kname = "fused_fwd_kernel" if args.path == "fused" else "alt_step_kernel"
    true_kib = args.copy_mib * 1024.0
    # the calibration copies are the last five copies of their run (a benchmark run with
    # --also-copy first copies its inputs to the device with the same copy kernel)
    fc, _, _ = _counter_mean(fetch_copy_csv, "copyBuffer", last=5)
    wc, _, _ = _counter_mean(write_copy_csv, "copyBuffer", last=5)
    fk, nf, names = _counter_mean(fetch_csv, kname)
    wk, nw, _ = _counter_mean(write_csv, kname)
    ff, wf = true_kib / fc, true_kib / wc
    w = fi.get_workload(args.workload)
    if args.backward:
        # the partial-sum serial kernel's own: the step records (8 floats a unit) read once, dWx
        # (fp32) and the dR operand da (bf16) of every gate written once, R read once
        alg = float(w.T * w.B * w.N * w.D * (8 * 4 + w.G * (4 + 2)) + w.G * w.N * w.D * w.D * 2)
    else:
        alg = headwise_bytes(w, 2 if "bf16" in w.name else 4)
    rd, wr = fk * 1024 * ff, wk * 1024 * wf
    entry = {"kernel": names[0], "dispatches": [nf, nw], "fetch_kib_per_dispatch": fk, "write_kib_per_dispatch": wk,
             "fetch_factor": ff, "write_factor": wf, "copy_mib": args.copy_mib, "read_bytes": rd, "write_bytes": wr,
             "bytes_per_launch": rd + wr, "algorithmic_bytes": alg, "kernel_sources_sha256_16": kernel_sources_hash()}
    try:
        with open(args.traffic_json) as f:
            allt = json.load(f)
    except (OSError, ValueError):
        allt = {}
    allt[f"{args.workload}:{args.path}" + (":backward" if args.backward else "")] = entry
    with open(args.traffic_json, "w") as f:
        json.dump(allt, f, indent=1)
        f.write("\n")
    print(json.dumps(entry))


def cpu_baseline(w, sample_T: int, backward: bool = False):
    """The oracle as it stands, on all (batch, head) rows for the first sample_T steps (the
    backward: its back-propagation through those steps, forward replay included)."""
    import numpy as np

    import frnn_inputs as fi
    import oracle

    x = fi.make_inputs(w)
    Wx = fi.to_f64(x["Wx"])[:, :sample_T]
    args = (Wx, fi.to_f64(x["R"]), fi.to_f64(x["b"]), fi.to_f64(x["states0"]))
    oracle.headwise_fwd(w.cell, Wx[:, :2], *args[1:])  # warm (loads the library)
    flops = 2.0 * w.B * w.N * w.G * w.D * w.D * sample_T
    t0 = time.perf_counter()
    if backward:
        ct = fi.backward_cotangents(w)
        oracle.headwise_bwd(w.cell, *args, fi.to_f64(ct["dstates"])[:, :, :sample_T], fi.to_f64(ct["dlast"]))
        flops = 2.0 * flops + 2.0 * (w.D + 1) * w.G * w.D * w.B * sample_T * w.N
    else:
        oracle.headwise_fwd(w.cell, *args)
    dt = time.perf_counter() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"all {w.B * w.N} (batch, head) rows x first {sample_T} of {w.T} timesteps, fp64, "
                      f"{dt:.2f} s wall" + (", backward" if backward else ""),
            "us_per_timestep": dt / sample_T * 1e6}


def measured_copy_gbs(mib: int = 256, reps: int = 10):
    """Bandwidth of a plain device-to-device copy of `mib` MiB (read + write bytes over the HIP-event
    time, the best of `reps`): the HBM roof this device reaches with a streaming kernel."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.randn(n, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    del src, dst
    return 2.0 * n * 4 / (best / 1e3) / 1e9


def engine_clock_under_load(step, seconds: float = 1.5, settle: float = 0.5):
    """The GPU engine clock (MHz) while `step` runs back to back: amd-smi's current graphics clock,
    sampled every 20 ms on the host while a queue of `seconds` of calls keeps the device busy,
    leaving out the first `settle` seconds (the clock ramps up and the firmware's figure lags);
    the median of the samples. None when amd-smi's Python module is not usable."""
    import threading

    import torch
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        handle = amdsmi.amdsmi_get_processor_handles()[torch.cuda.current_device()]
        amdsmi.amdsmi_get_clock_info(handle, amdsmi.AmdSmiClkType.GFX)
    except Exception:
        return None
    samples, done = [], threading.Event()

    def sample():
        t0 = time.perf_counter()
        while not done.is_set():
            try:
                clk = float(amdsmi.amdsmi_get_clock_info(handle, amdsmi.AmdSmiClkType.GFX)["clk"])
                if time.perf_counter() - t0 >= settle:
                    samples.append(clk)
            except Exception:
                pass
            time.sleep(0.02)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    step()
    e1.record()
    torch.cuda.synchronize()
    n = max(1, int(seconds / max(e0.elapsed_time(e1) / 1e3, 1e-6)))
    th = threading.Thread(target=sample)
    th.start()
    for _ in range(n):
        step()
    torch.cuda.synchronize()
    done.set()
    th.join()
    try:
        amdsmi.amdsmi_shut_down()
    except Exception:
        pass
    if len(samples) < 3:
        return None
    samples.sort()
    return samples[len(samples) // 2]


def calibration_copies(mib: int) -> None:
    """Five plain device-to-device copies of `mib` MiB (the known-size kernel the HBM counters are
    scaled by)."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.randn(n, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_mib": mib, "launches": 5,
                      "bytes_read_per_launch": n * 4, "bytes_written_per_launch": n * 4}), flush=True)


def sweep_designs(spec: str, T: int) -> None:
    """Pin every fused forward design through the planner's FRNN_FUSED_W / BR / NCW / KS variables,
    time each distinct design the planner accepts (the best of three calls after one warm-up,
    HIP events), and print its planner prediction beside the measurement; `pick` marks the design
    the planner chooses unpinned."""
    import re
    import torch
    import frnn_inputs as fi
    import head_wise_lstm_amd as hw
    cell, B, N, D = spec.split(",")
    B, N, D = int(B), int(N), int(D)
    pins = ["FRNN_FUSED_W", "FRNN_FUSED_BR", "FRNN_FUSED_NCW", "FRNN_FUSED_KS"]
    dev = torch.device("cuda:0")
    w = fi.HeadwiseWorkload("sweep", cell, torch.bfloat16, B=B, T=T, N=N, D=D, seed=0, s0_var=None)
    g = {k: (v.to(dev) if v is not None else None) for k, v in fi.make_inputs(w).items()}
    desc = hw._desc(B, T, N, D, cell, torch.bfloat16)

    def clear():
        for k in pins:
            os.environ.pop(k, None)

    def design(plan):
        m = dict(re.findall(r"(\w+)=(\S+)", plan))
        return ({"design": plan.split()[1].split("=")[1], **{k: int(m[k]) for k in
                 ("BR", "W", "NCW", "KS", "MTW", "KTW", "chunks")}}, float(m["predicted_us"]))

    def us_per_step():
        hw.frnn_fwd(g["Wx"], g["R"], g["b"], g["states0"], cell=cell, path="fused")
        torch.cuda.synchronize()
        ts = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            hw.frnn_fwd(g["Wx"], g["R"], g["b"], g["states0"], cell=cell, path="fused")
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return 1000.0 * min(ts) / T

    clear()
    pick, _ = design(hw.frnn_plan_str(desc))
    combos = [(1, br, ncw, 0) for br in range(1, 17) for ncw in (4, 8)]
    combos += [(W, br, ncw, ks) for W in range(2, 33) for br in range(1, 5)
               for ncw, ks in ((4, 1), (4, 2), (4, 4), (6, 6), (8, 2), (8, 4), (8, 8))]
    seen = []
    for W, br, ncw, ks in combos:
        clear()
        os.environ.update({"FRNN_FUSED_W": str(W), "FRNN_FUSED_BR": str(br), "FRNN_FUSED_NCW": str(ncw)})
        if ks:
            os.environ["FRNN_FUSED_KS"] = str(ks)
        try:
            d, pred = design(hw.frnn_plan_str(desc))
        except hw.FrnnError:
            continue
        if d in seen:
            continue
        seen.append(d)
        print(json.dumps({"shape": f"{cell}_B{B}_T{T}_N{N}_D{D}", **d, "predicted_us_per_call": pred,
                          "us_per_step": us_per_step(), "pick": d == pick}), flush=True)
    clear()


def ws_ring(nbytes: int, steps: int, dev):
    """Workspaces for the timed calls: one per call where they fit in WS_RING_BYTES (each call's
    error word then survives until it is checked), else as many as fit, at least one."""
    import torch
    k = max(1, min(steps, WS_RING_BYTES // max(nbytes, 1)))
    return [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(k)]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="lstm_bf16_B16_T1024_N1_D768")
    ap.add_argument("--path", default="fused", choices=["fused", "alternating"])
    ap.add_argument("--backward", action="store_true",
                    help="time frnn_bwd (back-propagation through time) instead of the forward: the "
                         "forward states are computed once before the timed region")
    ap.add_argument("--cpu-sample-T", type=int, default=0, help="timesteps of the CPU-baseline sample (0 = all)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (read MIB, write MIB), five times, for "
                         "scaling the HBM byte counters, and exit")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-roofs", action="store_true",
                    help="skip the engine-clock sample and the copy-bandwidth measurement after the timed region")
    ap.add_argument("--sweep-designs", default="", metavar="CELL,B,N,D",
                    help="time every fused forward design the planner can be pinned to on this head-wise shape "
                         "(bf16, seeded inputs, --sweep-T steps) and print one JSON line per design")
    ap.add_argument("--sweep-T", type=int, default=512)
    ap.add_argument("--also-copy", type=int, default=0, metavar="MIB",
                    help="after the benchmark, run the --copy-calibration copies in the same process, so that "
                         "one rocprofv3 counter pass records both")
    ap.add_argument("--write-traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "FETCH_COPY_CSV", "WRITE_COPY_CSV"),
                    help="only turn rocprofv3 FETCH_SIZE / WRITE_SIZE counter files of this workload and of "
                         "--copy-calibration into the --traffic-json entry, and exit (no GPU needed)")
    ap.add_argument("--copy-mib", type=int, default=256, help="size of the calibration copy (--write-traffic)")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="per-launch HBM bytes measured with rocprofv3 counters for this workload/path")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the recurrence is built for a single MI355X and this "
              f"build has no multi-GPU path (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        calibration_copies(args.copy_calibration)
        return
    if args.sweep_designs:
        sweep_designs(args.sweep_designs, args.sweep_T)
        return

    import frnn_inputs as fi
    import head_wise_lstm_amd as hw

    if not os.path.exists(hw.lib_path()):
        from head_wise_lstm_amd import build as hb
        hb.build(verbose=False)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    w = fi.get_workload(args.workload)
    x = fi.make_inputs(w)
    g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else ([t.to(dev) for t in v] if isinstance(v, list) else v))
         for k, v in x.items()}
    stream = torch.cuda.current_stream(dev)

    if isinstance(w, fi.HeadwiseWorkload):
        G, S = w.G, w.S
        desc = hw._desc(w.B, w.T, w.N, w.D, w.cell, w.dtype)
        wss = ws_ring(hw.frnn_workspace_bytes(desc, args.path), args.steps, dev)
        out = (torch.empty((S, w.B, w.T, w.N, w.D), dtype=torch.float32, device=dev),
               torch.empty((S, w.B, 1, w.N, w.D), dtype=torch.float32, device=dev))
        plan = hw.frnn_plan_str(desc, args.path)

        def step(i=0):
            hw.frnn_fwd(g["Wx"], g["R"], g["b"], g["states0"], cell=w.cell, path=args.path, out=out,
                        workspace=wss[i % len(wss)], check=False)
        flops = headwise_flops(w)
        if args.backward:
            fwd_st, _ = hw.frnn_fwd(g["Wx"], g["R"], g["b"], g["states0"], cell=w.cell, path="fused")
            ct = {k: v.to(dev) for k, v in fi.backward_cotangents(w).items()}
            wss = ws_ring(hw.frnn_bwd_workspace_bytes(desc, args.path), args.steps, dev)
            plan = hw.frnn_bwd_plan_str(desc, args.path)

            def step(i=0):
                hw.frnn_bwd(g["Wx"], g["R"], g["b"], g["states0"], fwd_st, ct["dstates"], ct["dlast"], cell=w.cell,
                            path=args.path, workspace=wss[i % len(wss)], check=False)
            # the serial contraction (da . R^T per step), the h.R recompute and the dR GEMM
            flops = 2.0 * headwise_flops(w) + 2.0 * (w.D + 1) * w.G * w.D * w.B * w.T * w.N
        elt = 2 if w.dtype == torch.bfloat16 else 4
        nbytes = headwise_bytes(w, elt)
        timesteps = w.T
        config = {"workload": w.name, "cell": w.cell, "B": w.B, "T": w.T, "N": w.N, "D": w.D, "G": G,
                  "in_dtype": str(w.dtype).replace("torch.", ""), "states_dtype": "float32", "path": args.path,
                  "plan": plan, "pass": "backward" if args.backward else "forward"}
        dtype = "bf16" if w.dtype == torch.bfloat16 else "f32"
    else:
        dirs = getattr(w, "dirs", 1)
        wss = ws_ring(hw.frnn_lstm_stack_workspace_bytes(w.L, w.T, w.B, w.I, w.H, args.path, dirs), args.steps, dev)
        out = (torch.empty((w.T, w.B, dirs * w.H), dtype=torch.float32, device=dev),
               torch.empty((w.L * dirs, w.B, w.H), dtype=torch.float32, device=dev),
               torch.empty((w.L * dirs, w.B, w.H), dtype=torch.float32, device=dev))

        def step(i=0):
            hw.frnn_lstm_stack_fwd(g["x"], g["Wi"], g["Wh"], g["b_ih"], g["b_hh"], g["h0"], g["c0"], path=args.path,
                                   out=out, workspace=wss[i % len(wss)], check=False, bidirectional=dirs == 2)
        flops = 2.0 * w.B * 4 * w.H * w.H * w.T * w.L * dirs  # recurrent contraction of all layers and directions
        if args.backward:
            ct = {k: v.to(dev) for k, v in fi.stack_cotangents(w).items()}
            wss = ws_ring(hw.frnn_lstm_stack_bwd_workspace_bytes(w.L, w.T, w.B, w.I, w.H, args.path, dirs), args.steps,
                          dev)

            def step(i=0):
                hw.frnn_lstm_stack_bwd(g["x"], g["Wi"], g["Wh"], g["b_ih"], g["b_hh"], g["h0"], g["c0"], ct["dout"],
                                       ct["dhn"], ct["dcn"], path=args.path, workspace=wss[i % len(wss)], check=False,
                                       bidirectional=dirs == 2)
            # forward again (recurrent contraction) + per layer the serial da.R^T, the h.R recompute
            # and the dR GEMM; the projections' GEMMs (forward, dWi, dX) are reported separately
            flops = 4.0 * flops
        nbytes = 0.0
        timesteps = w.T * w.L
        config = {"workload": w.name, "L": w.L, "dirs": dirs, "T": w.T, "B": w.B, "I": w.I, "H": w.H, "path": args.path,
                  "projection_gflop": (3.0 if args.backward else 1.0) * 2.0 * w.T * w.B * 4 * w.H * dirs *
                  (w.I + dirs * w.H * (w.L - 1)) / 1e9,
                  "pass": "backward" if args.backward else "forward"}
        if args.backward:  # each layer's serial part: the head-wise backward of one head of H units
            config["plan"] = hw.frnn_bwd_plan_str(hw._desc(w.B, w.T, 1, w.H, "lstm", w.dtype), args.path)
        dtype = "bf16"

    for i in range(args.warmup):
        step(i)
    for ws in wss:
        hw.frnn_check(ws)
    torch.cuda.synchronize()
    # one event between consecutive calls: the whole region's time and every call's own
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step(i)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # each call's device-side error word (a bounded wait that ran out, a workgroup on the wrong die)
    for ws in wss:
        hw.frnn_check(ws)
    ms = ev[0].elapsed_time(ev[-1]) / args.steps
    per_call = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    ms_median = per_call[len(per_call) // 2] if len(per_call) % 2 else 0.5 * (per_call[len(per_call) // 2 - 1] +
                                                                                per_call[len(per_call) // 2])
    ms_min = per_call[0]
    sec = ms / 1e3
    tflops = flops / sec / 1e12
    roof = {"bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": tflops / PEAK_BF16_TFLOPS, "traffic": None,
            "kernel": ((("frnn::fused_bwdx_kernel" if "die-local-partials" in str(config.get("plan", "")) else
                         "frnn::fused_bwd_local_kernel" if "workgroup-local" in str(config.get("plan", "")) else
                         "frnn::fused_bwd_kernel") + " (+ GEMMs, records)" if args.path == "fused" else
                        "frnn::bwd_gate_kernel+bwd_dh_kernel (+ GEMMs)") if args.backward else
                       "frnn::fused_fwd_kernel" if args.path == "fused" else "frnn::alt_step_kernel"),
            "per_launch_flop": flops, "launch_ms": ms}
    if not args.no_roofs:
        clk = engine_clock_under_load(step)
        roof["engine_clock_mhz"] = clk
        roof["frac_at_measured_clock"] = None if not clk else tflops / (PEAK_BF16_TFLOPS * clk / PEAK_SCLK_MHZ)
        roof["measured_copy_gbs"] = measured_copy_gbs()
    if nbytes and not args.backward:
        roof["algorithmic_bytes"] = nbytes
        roof["hbm_frac"] = nbytes / sec / 1e9 / PEAK_HBM_GBS
    # HBM bytes per launch counted by rocprofv3 (FETCH_SIZE + WRITE_SIZE, calibrated on a plain
    # copy), valid only for the kernel source they were taken on
    try:
        with open(args.traffic_json) as f:
            tj = json.load(f).get(f"{config['workload']}:{args.path}" + (":backward" if args.backward else ""))
        if tj and tj.get("kernel_sources_sha256_16") == kernel_sources_hash():
            roof["traffic"] = tj["bytes_per_launch"]
            roof["traffic_over_algorithmic"] = tj["bytes_per_launch"] / tj["algorithmic_bytes"]
    except (OSError, ValueError, KeyError):
        pass
    if args.backward:
        metric = f"{w.name} backward achieved TFLOP/s (serial contraction, h.R recompute and dR GEMM)"
    elif w.name == fi.HEADLINE:
        metric = METRIC
    else:
        metric = f"{w.name} fwd achieved TFLOP/s of the recurrent contraction"
    res = {"metric": metric, "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": dtype, "data": "synthetic (seeded, shapes and distributions of the workload)",
           "config": config, "us_per_timestep": ms * 1e3 / timesteps,
           "ms_per_call_median": ms_median, "ms_per_call_min": ms_min,
           "us_per_timestep_median": ms_median * 1e3 / timesteps, "us_per_timestep_min": ms_min * 1e3 / timesteps,
           "calls_error_checked": min(len(wss), args.steps),
           "pct_mfma_bf16_peak": 100.0 * tflops / PEAK_BF16_TFLOPS, "wall_s_timed": wall, "roofline": roof}
    if not args.no_cpu_baseline and isinstance(w, fi.HeadwiseWorkload):
        res["cpu_baseline"] = cpu_baseline(w, min(args.cpu_sample_T or w.T, w.T), backward=args.backward)
    print(json.dumps(res), flush=True)
    if args.also_copy:
        calibration_copies(args.also_copy)


if __name__ == "__main__":
    main()
