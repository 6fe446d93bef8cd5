"""Build the CPU oracle library (test infrastructure only).

    python oracle/build.py [-v] [--sanitize]

Compiles gdr_oracle.c with gcc into oracle/libgdr_oracle.so: -O2, contraction
off and no fast-math, so every multiply and add rounds exactly as written.

--sanitize builds oracle/libgdr_oracle_sanitize.so instead, the same source
with AddressSanitizer and UndefinedBehaviorSanitizer (host code only; the
oracle has no GPU code).  Run the oracle's CPU tests against it with

    GDR_ORACLE_LIB=oracle/libgdr_oracle_sanitize.so \\
    LD_PRELOAD="$(gcc -print-file-name=libasan.so) $(gcc -print-file-name=libubsan.so)" \\
    ASAN_OPTIONS=detect_leaks=0 UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1 \\
    python -m pytest tests/test_oracle_pins.py tests/test_oracle_sweep.py \\
        tests/test_oracle_threads.py -q

(leak detection is off because the Python interpreter itself holds memory
until exit; the oracle frees everything it allocates).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gdr_oracle.c")
LIB = os.path.join(HERE, "libgdr_oracle.so")
SANITIZE_LIB = os.path.join(HERE, "libgdr_oracle_sanitize.so")

CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fno-strict-aliasing",
          "-Wall", "-Wextra", "-shared", "-fPIC", "-pthread"]
SANITIZE_FLAGS = ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=undefined"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    out = SANITIZE_LIB if sanitize else LIB
    cmd = ["gcc", *CFLAGS, *(SANITIZE_FLAGS if sanitize else []), SRC, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
