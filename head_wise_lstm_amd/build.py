"""Compile libfrnn.so (gfx950) in-tree with hipcc.

Usage: python -m head_wise_lstm_amd.build   (or head_wise_lstm_amd.build.build()).
"""
from __future__ import annotations

import os
import subprocess
import sys
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
    "-shared",
    # keep packed-fp32 VALU instructions out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def build(verbose: bool = True) -> str:
    src = os.path.join(CSRC, "frnn_api.hip")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, src, "-o", tmp]
    t0 = time.time()
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature; that is expected.
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if res.returncode != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError("hipcc failed building libfrnn.so")
    if verbose and msgs:
        print("\n".join(msgs[:40]))
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f}s", flush=True)
    return LIB


if __name__ == "__main__":
    build()
