"""The C ABI used from a plain HIP host program, with no Python binding and
no torch in the process (tests/c_abi/consumer.cpp, built by build()): a ragged
forward against the CPU oracle and an argument error reported before any
launch."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "consumer")


def test_c_consumer_without_python_binding():
    assert os.path.exists(BIN), "tests/c_abi/consumer is not built (run __graft_entry__.build())"
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout.strip(), flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "other slots untouched" in r.stdout
