"""The optional index checks on the CPU: gdr_check_indices on host arrays
reports every violation of the index preconditions (decreasing offsets,
offsets past the tokens, out-of-range or repeated slots, out-of-range or
shared ring rows among the rows that use the ring) with GDR_ERR_INVALID_ARG
and a message, and accepts what the kernels allow (padding rows, repeated
padding, ring rows of rows that do not use the ring)."""
import os

import numpy as np
import pytest

from gated_delta_rule_loop_amd import _binding as B

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH),
                                reason="libgdr.so not built (run __graft_entry__.build())")

PAD = 0xFFFFFFFF
u32 = lambda *a: np.array(a, dtype=np.uint32)  # noqa: E731


def rejects(match, **kw):
    with pytest.raises(B.GdrError) as e:
        B.gdr_check_indices(**kw)
    assert e.value.code == -1
    assert match in str(e.value), str(e.value)


def test_valid_indices_pass():
    B.gdr_check_indices(4, row_offsets=u32(0, 3, 3, 9, 10), total_tokens=10,
                        slots=u32(5, PAD, 0, PAD), num_slots=6,
                        ring_idx=u32(1, 1, 0, 7), ring_rows=2, ring_len=8)
    # int32 indices with -1 padding are the same bits
    B.gdr_check_indices(3, slots=np.array([2, -1, -1], np.int32), num_slots=3)
    # offsets may end before the tokens (trailing tokens belong to no row)
    B.gdr_check_indices(2, row_offsets=u32(2, 4, 6), total_tokens=9)
    assert B.lib().gdr_last_error_message() == b""


def test_offsets():
    rejects("decrease at row 1", rows=3, row_offsets=u32(0, 4, 3, 8), total_tokens=8)
    rejects("past the 8 tokens", rows=2, row_offsets=u32(0, 4, 9), total_tokens=8)


def test_slots():
    rejects("slot 6 of row 1 is not below the 6", rows=2, slots=u32(0, 6), num_slots=6)
    rejects("slot 3 is used by rows 0 and 2", rows=3, slots=u32(3, 1, 3), num_slots=6)
    rejects("is used by rows", rows=2, slots=np.array([4, 4], np.int32), num_slots=6)


def test_verify_ring_rows():
    off = u32(0, 2, 14, 17)          # lengths 2, 12, 3 with ring_len 8: row 1 commits
    ok = dict(rows=3, row_offsets=off, total_tokens=17, slots=u32(0, 1, 2), num_slots=3,
              ring_rows=4, ring_len=8)
    B.gdr_check_indices(ring_idx=u32(0, 9, 1), **ok)    # row 1 records nothing
    B.gdr_check_indices(ring_idx=u32(0, 0, 1), **dict(ok, slots=u32(0, 1, 2)))
    rejects("ring row 4 of row 2 is not below the 4", ring_idx=u32(0, 0, 4), **ok)
    rejects("ring row 3 is used by rows 0 and 2", ring_idx=u32(3, 1, 3), **ok)
    # a padding row does not use the ring; an empty row records nothing either
    B.gdr_check_indices(ring_idx=u32(3, 1, 3), **dict(ok, slots=u32(0, 1, PAD)))
    B.gdr_check_indices(rows=2, row_offsets=u32(0, 0, 3), total_tokens=3, slots=u32(0, 1),
                        num_slots=2, ring_idx=u32(2, 2), ring_rows=3, ring_len=8)


def test_fold_ring_rows():
    ok = dict(rows=3, slots=u32(0, 1, 2), num_slots=3, ring_rows=4, ring_len=8)
    # accepted 0 and > ring_len leave the row alone: its ring row is unused
    B.gdr_check_indices(ring_idx=u32(9, 1, 9), accepted=u32(0, 5, 11), **ok)
    rejects("ring row 9 of row 1", ring_idx=u32(0, 9, 1), accepted=u32(1, 5, 2), **ok)
    rejects("ring row 1 is used by rows 1 and 2", ring_idx=u32(0, 1, 1),
            accepted=u32(1, 5, 2), **ok)


def test_debug_switch_round_trip():
    before = B.gdr_set_debug_checks(True)
    try:
        assert B.gdr_set_debug_checks(False) is True
        assert B.gdr_set_debug_checks(False) is False
    finally:
        B.gdr_set_debug_checks(before)
