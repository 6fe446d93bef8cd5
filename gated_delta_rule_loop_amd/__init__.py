"""gated_delta_rule_loop_amd - the gated delta rule recurrence on MI355X (gfx950).

The computation lives in libgdr.so (hand-written HIP kernels behind the C ABI
of include/gdr.h).  This package is its thin binding: the functions below
marshal torch device tensors into the C ABI and nothing else.  Build the
library with `python -m gated_delta_rule_loop_amd.build`.
"""
from ._binding import (  # noqa: F401
    GdrError,
    gdr_causal_conv1d,
    gdr_check_indices,
    gdr_fused_recurrent_update,
    gdr_fwd_output_shape,
    gdr_last_error_message,
    gdr_recurrence_fwd,
    gdr_recurrence_verify_ring,
    gdr_set_debug_checks,
    gdr_ring_record_elements,
    gdr_snapshot_rollback,
    gdr_state_fold,
    gdr_version,
    lib,
)
