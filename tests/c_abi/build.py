"""Build the C-ABI consumer test program (tests/c_abi/consumer).

    python tests/c_abi/build.py

A host program compiled by hipcc for gfx950 that links libgdr.so and the CPU
oracle library, both found next to it at run time through $ORIGIN-relative
run paths, so the built tree works wherever it is copied.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "consumer.cpp")
BIN = os.path.join(HERE, "consumer")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False) -> str:
    pkg = os.path.join(ROOT, "gated_delta_rule_loop_amd")
    orc = os.path.join(ROOT, "oracle")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", "-Wall",
           "-I", os.path.join(ROOT, "include"), SRC,
           "-L", pkg, "-lgdr", "-L", orc, "-lgdr_oracle",
           "-Wl,-rpath,$ORIGIN/../../gated_delta_rule_loop_amd",
           "-Wl,-rpath,$ORIGIN/../../oracle", "-o", BIN + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(BIN + ".tmp", BIN)
    return BIN


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
