"""Build the HIP library libgdr.so in-tree for gfx950.

    python -m gated_delta_rule_loop_amd.build [-v]

Every source is compiled by hipcc for gfx950 only, with contraction off (the
kernels spell out each fused multiply-add they want, which keeps the forward,
verify and fold kernels bit-identical) and packed-fp32 VALU instructions
disabled.  The recurrence tables (one per work type, state type and kernel
mode) are separate translation units, compiled in parallel, then linked.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgdr.so")
SOURCES = [os.path.join(CSRC, "gdr_api.cpp"), os.path.join(CSRC, "gdr_kernels.hip"),
           os.path.join(CSRC, "gdr_conv.hip")]
TABLE_SOURCE = os.path.join(CSRC, "gdr_rec_table.hip")
# (work type, state storage type, kernel mode) of each recurrence table:
# types float or uint16_t (bf16 bits); modes kPlain 0, kVerify 1, kSnap 2,
# plus kBetaCols 4 (per-column beta).
TABLES = [(wt, st, mode) for wt in ("float", "uint16_t") for st in ("uint16_t", "float")
          for mode in (0, 1, 2, 4, 6)]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]
_NOISE = "is not a recognized feature for this target"


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(line for line in res.stderr.splitlines() if _NOISE not in line)
    return res.returncode, err


def compile_commands(objdir, defines=()):
    """(object, hipcc command) of every translation unit."""
    jobs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        jobs.append((obj, [HIPCC, *FLAGS, *defines, "-x", "hip", "-c", src, "-o", obj]))
    for wt, st, mode in TABLES:
        obj = os.path.join(objdir, f"table_{wt}_{st}_{mode}.o")
        jobs.append((obj, [HIPCC, *FLAGS, *defines, f"-DGDR_WT={wt}", f"-DGDR_ST={st}",
                           f"-DGDR_MODE={mode}", "-x", "hip", "-c", TABLE_SOURCE, "-o", obj]))
    return jobs


def build(verbose: bool = False, defines=(), out: str = LIB, jobs: int | None = None) -> str:
    """Compile every translation unit in parallel and link libgdr.so."""
    jobs = jobs or min(len(TABLES) + len(SOURCES), os.cpu_count() or 4)
    with tempfile.TemporaryDirectory(prefix="gdr_build_") as objdir:
        units = compile_commands(objdir, defines)
        if verbose:
            for _, cmd in units:
                print(" ".join(cmd), flush=True)
        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(lambda u: _run(u[1]), units))
        for (obj, _), (rc, err) in zip(units, results):
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {os.path.basename(obj)} ({rc}):\n{err}")
            if verbose and err.strip():
                print(err)
        tmp = out + ".tmp"
        rc, err = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC",
                        *[obj for obj, _ in units], "-o", tmp])
        if rc != 0:
            raise RuntimeError(f"link failed ({rc}):\n{err}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
