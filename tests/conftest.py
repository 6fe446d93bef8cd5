import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (HIP device); parity tests proper")


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    """The CPU oracle is test infrastructure; build it if it is missing."""
    lib = os.path.join(ROOT, "oracle", "libgdr_oracle.so")
    if not os.path.exists(lib):
        from oracle import build
        build.build()
    yield


def pytest_terminal_summary(terminalreporter):
    """One line that survives -q: the bf16 rounding ties the GPU parity tests
    accepted, against every bf16 element they compared with the oracle."""
    harness = sys.modules.get("tests.gpu_harness")
    if harness is None or not harness.TIE_STATS["comparisons"]:
        return
    t = harness.TIE_STATS
    terminalreporter.write_line(
        f"bf16 ties: {t['ties']} of {t['elements']} bf16 elements compared with the oracle "
        f"({t['comparisons']} comparisons; largest tie offset from the midpoint "
        f"{t['max_tie_offset']:.1e} of max|ref|, margin {harness.FLIP_MARGIN:.0e})")
    if harness.FP32_GAPS:
        gaps = ", ".join(f"{k} {v:.1e}" for k, v in harness.FP32_GAPS.items())
        terminalreporter.write_line(f"float32 state gap GPU vs oracle (of max|ref|): {gaps}")
