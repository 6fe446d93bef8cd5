"""The oracle's work-item farm: running the independent (row, value head)
items on several threads gives the single-threaded results bit for bit, and an
item's error still reaches the caller (CPU only)."""
import numpy as np
import pytest

import oracle
from gated_delta_rule_loop_amd import workloads as wl


def _ragged(seed, lengths, nk=2, nv=4, K=16, V=16, pad_rows=(1,)):
    rng = np.random.Generator(np.random.PCG64(seed))
    return wl.packed_inputs(rng, lengths, nk=nk, nv=nv, K=K, V=V, slots=12, state_dtype="bf16",
                            state_sigma=0.1, pad_rows=pad_rows)


def _fwd(w, threads):
    return oracle.recurrence_fwd(**{k: w[k] for k in (
        "qkv", "decay", "beta", "state", "slot_idx", "row_offsets", "num_value_heads",
        "num_key_heads")}, threads=threads)


@pytest.mark.parametrize("threads", [2, 3, 8])
def test_threaded_forward_is_bit_identical(threads):
    w = _ragged(7, [5, 3, 0, 17, 1, 9, 2])
    out1, st1 = _fwd(w, 1)
    outn, stn = _fwd(w, threads)
    assert np.array_equal(out1.view(np.uint32), outn.view(np.uint32))
    assert np.array_equal(st1, stn)


def test_threaded_verify_is_bit_identical():
    w = _ragged(8, [5, 3, 11, 1, 9, 2])
    stride = wl.ring_record_stride(2, 16, 16)
    args = {k: w[k] for k in ("qkv", "decay", "beta", "state", "slot_idx", "row_offsets",
                              "num_value_heads", "num_key_heads")}
    args["ring"] = np.zeros((8, 2, 8, stride), np.float32)
    args["ring_slot_idx"] = np.array([7, 0, 3, 5, 1, 2], np.uint32)
    o1, s1, r1 = oracle.recurrence_verify_ring(**args, threads=1)
    o4, s4, r4 = oracle.recurrence_verify_ring(**args, threads=4)
    assert np.array_equal(o1.view(np.uint32), o4.view(np.uint32))
    assert np.array_equal(s1, s4)
    assert np.array_equal(r1.view(np.uint32), r4.view(np.uint32))


def test_threaded_fused_update_is_bit_identical():
    rng = np.random.Generator(np.random.PCG64(9))
    w = wl.gdp_inputs(rng, B=6, S_draft=3, M=2, H=2, HV=4, K=16, V=32, slots=10,
                      pad_frac=0.2, state_sigma=0.05)
    r1 = oracle.fused_recurrent_update(**w, threads=1)
    r5 = oracle.fused_recurrent_update(**w, threads=5)
    for a, b in zip(r1, r5):
        assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))


def test_threaded_error_reaches_the_caller():
    w = _ragged(10, [2, 3, 4], pad_rows=())
    w["slot_idx"] = np.array([0, 99, 1], np.uint32)  # 99 is past the 12-slot pool
    with pytest.raises(ValueError):
        _fwd(w, 4)


def test_default_threads_is_positive():
    assert oracle.default_threads() >= 1
