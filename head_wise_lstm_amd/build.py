"""Compile libfrnn.so (gfx950) in-tree with hipcc.

Usage: python -m head_wise_lstm_amd.build   (or head_wise_lstm_amd.build.build()).
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfrnn.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # keep packed-fp32 VALU instructions out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


# Translation units: the host side with the small kernels, and the fused kernel's instantiations
# for each cell (the slow part, so they compile in parallel).
SOURCES = ["frnn_api.hip", "frnn_fused_lstm.hip", "frnn_fused_elman.hip", "frnn_fused_gru.hip"]


def _messages(res) -> list:
    # hipcc's host pass warns that it does not know the packed-fp32 feature; that is expected.
    return [l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l and l.strip()]


def build(verbose: bool = True) -> str:
    t0 = time.time()
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    with tempfile.TemporaryDirectory(prefix="frnn_build_") as tmpdir:
        procs, objs = [], []
        for src in SOURCES:
            obj = os.path.join(tmpdir, os.path.splitext(src)[0] + ".o")
            cmd = [HIPCC, *FLAGS, "-c", *inc, os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
            objs.append(obj)
        failed = []
        for src, pr in procs:
            out, err = pr.communicate()
            res = subprocess.CompletedProcess(pr.args, pr.returncode, out, err)
            msgs = _messages(res)
            if pr.returncode != 0:
                sys.stderr.write("\n".join(msgs) + "\n")
                failed.append(src)
            elif verbose and msgs:
                print("\n".join(msgs[:40]))
        if failed:
            raise RuntimeError("hipcc failed building " + ", ".join(failed))
        tmp = LIB + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write("\n".join(_messages(res)) + "\n")
            raise RuntimeError("linking libfrnn.so failed")
        os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f}s", flush=True)
    return LIB


if __name__ == "__main__":
    build()
