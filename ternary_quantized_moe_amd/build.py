"""Build libmoe_ternary.so in-tree with hipcc for gfx950.

    python -m ternary_quantized_moe_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoe_ternary.so")
SOURCES = ["moe_capi.hip", "moe_kernels.hip", "moe_experts.hip", "moe_dense.hip", "moe_quant.hip", "moe_ple.hip", "moe_mtp.hip", "moe_router_delta.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = True) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln and ln.strip()]
    if msgs and verbose:
        sys.stderr.write("\n".join(msgs) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
