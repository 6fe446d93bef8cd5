"""Build the CPU oracle library (test infrastructure only).

    python oracle/build.py

Compiles gdr_oracle.c with gcc into oracle/libgdr_oracle.so: -O2, contraction
off and no fast-math, so every multiply and add rounds exactly as written.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gdr_oracle.c")
LIB = os.path.join(HERE, "libgdr_oracle.so")

CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fno-strict-aliasing",
          "-Wall", "-Wextra", "-shared", "-fPIC", "-pthread"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
