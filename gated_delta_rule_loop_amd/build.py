"""Build the HIP library libgdr.so in-tree for gfx950.

    python -m gated_delta_rule_loop_amd.build [-v]

Every source is compiled by hipcc for gfx950 only, with contraction off (the
kernels spell out each fused multiply-add they want, which keeps the forward,
verify and fold kernels bit-identical) and packed-fp32 VALU instructions
disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgdr.so")
SOURCES = [os.path.join(CSRC, "gdr_api.cpp"), os.path.join(CSRC, "gdr_kernels.hip")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def build(verbose: bool = False) -> str:
    out = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-x", "hip", *SOURCES, "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in res.stderr.splitlines() if noise not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err)
    os.replace(out, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
