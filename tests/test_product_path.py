"""The product path has no CPU fallback and never reaches the oracle (CPU
only): the package and the HIP sources name no oracle module or symbol, and
the binding raises instead of computing when libgdr.so is missing."""
import os
import re

import pytest

import gated_delta_rule_loop_amd
from gated_delta_rule_loop_amd import _binding as B

PKG = os.path.dirname(gated_delta_rule_loop_amd.__file__)


def _sources():
    for root, _, files in os.walk(PKG):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                yield os.path.join(root, f)


def test_package_never_imports_the_oracle():
    hits = []
    for path in _sources():
        text = open(path).read()
        if re.search(r"^\s*(import|from)\s+oracle\b|gdr_oracle|oracle_recurrence", text, re.M):
            hits.append(path)
    assert not hits, f"product sources reach the oracle: {hits}"


def test_missing_library_raises_instead_of_falling_back(monkeypatch):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", os.path.join(PKG, "no_such_libgdr.so"))
    with pytest.raises(ImportError):
        B.lib()
    with pytest.raises(ImportError):
        B.gdr_ring_record_elements(2, 128, 128)
