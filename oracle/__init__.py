"""Python access to the plain CPU oracle (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It wraps oracle/gdr_oracle.c (built by oracle/build.py) with
ctypes and works on NumPy arrays.  bfloat16 tensors are carried as uint16 bit
patterns.  Every function copies its state-like inputs and returns new arrays;
the caller's arrays are never written.

Sources: the four documentation pages "gated_delta_recurrence_fwd_gpu",
"gated_delta_recurrence_verify_ring_gpu", "gated_delta_recurrence_fwd_shape"
and "core.ssm.ops.gdp.fused_recurrent"; see gdr_oracle.c for which part of
which page each function follows.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# GDR_ORACLE_LIB selects another build of gdr_oracle.c (the sanitizer build
# of oracle/build.py --sanitize); the default is the plain build.
_LIB_PATH = os.environ.get("GDR_ORACLE_LIB") or os.path.join(_HERE, "libgdr_oracle.so")
_lib = None

PAD_SLOT = 0xFFFFFFFF

_ENTRY_POINTS = ("oracle_recurrence_fwd_threads", "oracle_recurrence_verify_ring_threads",
                 "oracle_state_fold", "oracle_fused_recurrent_update_threads",
                 "oracle_snapshot_rollback", "oracle_causal_conv1d")


def default_threads() -> int:
    """Threads for the work-item farm: OMP_NUM_THREADS if set, else the CPUs
    this process may run on."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover - non-Linux
        return max(1, os.cpu_count() or 1)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build  # noqa: PLC0415
            _build.build()
        _lib = ctypes.CDLL(_LIB_PATH)
        for name in _ENTRY_POINTS:
            getattr(_lib, name).restype = ctypes.c_int
    return _lib


class using_library:
    """Context manager: route the functions below through another build of
    gdr_oracle.c (the tests use it to run the pins against planted mistakes)."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = _load()
        lib = ctypes.CDLL(self.path)
        for name in _ENTRY_POINTS:
            getattr(lib, name).restype = ctypes.c_int
        _lib = lib
        return lib

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


def _state_copy(a):
    """Copy a state-like array; returns (copy, is_bf16)."""
    if a is None:
        return None, 0
    if a.dtype == np.uint16:
        return np.array(a, dtype=np.uint16, order="C", copy=True), 1
    if a.dtype == np.float32:
        return np.array(a, dtype=np.float32, order="C", copy=True), 0
    raise TypeError(f"state arrays must be float32 or uint16 (bf16 bits), got {a.dtype}")


def _work(arrays):
    """Per-token inputs of one call: all float32, or all uint16 (bf16 bits),
    the work dtype.  Returns (float32 arrays, is_bf16); bf16 widens exactly."""
    kinds = {a.dtype for a in arrays if a is not None}
    if len(kinds) > 1:
        raise TypeError("per-token inputs must share one work dtype")
    bf = kinds == {np.dtype(np.uint16)}
    conv = []
    for a in arrays:
        if a is None:
            conv.append(None)
        elif bf:
            b = np.ascontiguousarray(a, dtype=np.uint16).astype(np.uint32) << 16
            conv.append(b.view(np.float32))
        else:
            conv.append(np.ascontiguousarray(a, dtype=np.float32))
    return conv, bf


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, nearest even (the oracle's own rounding)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_bf16_round_array(_p(x), _p(out), ctypes.c_int64(x.size))
    return out


def default_scale(K: int) -> float:
    return 1.0 / math.sqrt(K)


def recurrence_fwd(*, qkv, decay, beta, state, slot_idx, row_offsets, num_value_heads,
                   num_key_heads, scale=None, l2norm=True, threads=1):
    """Ragged slot-indexed forward ("gated_delta_recurrence_fwd_gpu").

    qkv, decay and beta share the work dtype: float32, or uint16 bf16 bits
    (verify page, work_dtype), which widen exactly; the output is then rounded
    to bf16 once.  threads > 1 runs the independent (row, value head) items
    on that many threads (same results).  Returns (out [T, nv*V] of the work
    dtype, state_after)."""
    lib = _load()
    st, bf = _state_copy(state)
    K, V = st.shape[2], st.shape[3]
    (qkv, decay, beta), work_bf16 = _work((qkv, decay, beta))
    off = np.ascontiguousarray(row_offsets, dtype=np.uint32)
    sl = np.ascontiguousarray(slot_idx, dtype=np.uint32)
    B = sl.shape[0]
    T = qkv.shape[0]
    out = np.zeros((T, num_value_heads * V), dtype=np.float32)
    sc = default_scale(K) if scale is None else scale
    rc = lib.oracle_recurrence_fwd_threads(
        B, num_value_heads, num_key_heads, K, V, _p(off), _p(sl), _p(qkv), _p(decay), _p(beta),
        bf, _p(st), ctypes.c_int64(st.shape[0]), _p(out), ctypes.c_float(sc), int(l2norm),
        int(threads))
    if rc != 0:
        raise ValueError(f"oracle_recurrence_fwd failed: {rc}")
    return (bf16_round(out) if work_bf16 else out), st


def recurrence_fwd_into(*, out, state, qkv, decay, beta, slot_idx, row_offsets,
                        num_value_heads, num_key_heads, scale=None, l2norm=True, threads=1):
    """recurrence_fwd writing into the caller's arrays: out [T, nv*V] float32
    and the pool state (float32 or uint16 bf16 bits), both C-contiguous and
    updated in place; float32 per-token inputs only.  For timing the oracle
    itself (no copy of the pool per call)."""
    lib = _load()
    if state.dtype not in (np.float32, np.uint16) or out.dtype != np.float32:
        raise TypeError("state must be float32 or uint16, out float32")
    for a in (qkv, decay, beta):
        if a.dtype != np.float32:
            raise TypeError("per-token inputs must be float32")
    K, V = state.shape[2], state.shape[3]
    off = np.ascontiguousarray(row_offsets, dtype=np.uint32)
    sl = np.ascontiguousarray(slot_idx, dtype=np.uint32)
    sc = default_scale(K) if scale is None else scale
    rc = lib.oracle_recurrence_fwd_threads(
        sl.shape[0], num_value_heads, num_key_heads, K, V, _p(off), _p(sl), _p(qkv),
        _p(decay), _p(beta), int(state.dtype == np.uint16), _p(state),
        ctypes.c_int64(state.shape[0]), _p(out), ctypes.c_float(sc), int(l2norm), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_recurrence_fwd failed: {rc}")


def ring_record_elements(group: int, K: int, V: int) -> int:
    """Elements of one ring record: k_hat, then u and a of each of the group's
    value heads."""
    return K + group * (V + 1)


def recurrence_verify_ring(*, qkv, decay, beta, state, slot_idx, row_offsets, num_value_heads,
                           num_key_heads, ring, ring_slot_idx, scale=None, l2norm=True,
                           threads=1):
    """Verify window with ring ("gated_delta_recurrence_verify_ring_gpu").

    ring: [ring_rows, nk, ring_len, rec_stride], float32 or uint16 (bf16 bits),
    copied.  Work dtype and threads as recurrence_fwd.
    Returns (out, state_after, ring_after)."""
    lib = _load()
    st, bf = _state_copy(state)
    K, V = st.shape[2], st.shape[3]
    (qkv, decay, beta), work_bf16 = _work((qkv, decay, beta))
    off = np.ascontiguousarray(row_offsets, dtype=np.uint32)
    sl = np.ascontiguousarray(slot_idx, dtype=np.uint32)
    rsl = np.ascontiguousarray(ring_slot_idx, dtype=np.uint32)
    rg, rbf = _state_copy(ring)
    B, T = sl.shape[0], qkv.shape[0]
    out = np.zeros((T, num_value_heads * V), dtype=np.float32)
    sc = default_scale(K) if scale is None else scale
    rc = lib.oracle_recurrence_verify_ring_threads(
        B, num_value_heads, num_key_heads, K, V, _p(off), _p(sl), _p(qkv), _p(decay), _p(beta),
        bf, _p(st), ctypes.c_int64(st.shape[0]), _p(out), ctypes.c_float(sc), int(l2norm),
        _p(rg), rbf, _p(rsl), ctypes.c_int64(rg.shape[0]), rg.shape[2],
        ctypes.c_int64(rg.shape[3]), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_recurrence_verify_ring failed: {rc}")
    return (bf16_round(out) if work_bf16 else out), st, rg


def state_fold(*, state, slot_idx, ring, ring_slot_idx, accepted, num_value_heads,
               num_key_heads):
    """Fold the first accepted[b] ring records of each row into its state.

    Returns state_after."""
    lib = _load()
    st, bf = _state_copy(state)
    K, V = st.shape[2], st.shape[3]
    rg = np.ascontiguousarray(ring)
    if rg.dtype not in (np.float32, np.uint16):
        raise TypeError("ring must be float32 or uint16 (bf16 bits)")
    rbf = int(rg.dtype == np.uint16)
    sl = np.ascontiguousarray(slot_idx, dtype=np.uint32)
    rsl = np.ascontiguousarray(ring_slot_idx, dtype=np.uint32)
    acc = np.ascontiguousarray(accepted, dtype=np.uint32)
    rc = lib.oracle_state_fold(
        sl.shape[0], num_value_heads, num_key_heads, K, V, _p(sl), bf, _p(st),
        ctypes.c_int64(st.shape[0]), _p(rg), rbf, _p(rsl), ctypes.c_int64(rg.shape[0]),
        rg.shape[2], ctypes.c_int64(rg.shape[3]), _p(acc))
    if rc != 0:
        raise ValueError(f"oracle_state_fold failed: {rc}")
    return st


def fused_recurrent_update(*, q, k, v, g=None, beta=None, scale=None, initial_state=None,
                           output_final_state=False, use_qk_l2norm_in_kernel=False,
                           cu_seqlens=None, state=None, state_indices=None,
                           intermediate_states=None, steps_per_token=1, threads=1):
    """Fused recurrent update ("core.ssm.ops.gdp.fused_recurrent").

    q, k [B, T, H, K]; v [B, T, HV, V]; g, beta [B, T, HV] (beta may be
    [B, T, HV, V]); state [S, HV, K, V]; intermediate_states [S, T//spt, HV, K, V].
    State-like arrays are float32 or uint16 (bf16 bits) and must share a dtype;
    q, k, v, g, beta share the work dtype likewise, and o is of that dtype.
    Returns (o, final_state, intermediate_after): final_state is the updated
    pool copy when a pool is given, the dense final state when requested, else
    None; intermediate_after is the updated snapshot copy or None.  threads as
    recurrence_fwd (items are (sequence, value head) pairs)."""
    lib = _load()
    (q, k, v, g, beta), work_bf16 = _work((q, k, v, g, beta))
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    beta_per_v = int(beta is not None and beta.ndim == 4)
    cu = None if cu_seqlens is None else np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    N = B if cu is None else cu.shape[0] - 1
    st, bf = _state_copy(state)
    init, bf_i = _state_copy(initial_state)
    inter, bf_m = _state_copy(intermediate_states)
    dtypes = {x for x, arr in ((bf, st), (bf_i, init), (bf_m, inter)) if arr is not None}
    if len(dtypes) > 1:
        raise TypeError("state-like arrays must share one dtype")
    sbf = dtypes.pop() if dtypes else 0
    final = None
    if st is None and output_final_state:
        final = np.zeros((N, HV, K, V), dtype=np.uint16 if sbf else np.float32)
    idx = None if state_indices is None else np.ascontiguousarray(state_indices, dtype=np.int32)
    o = np.zeros((B, T, HV, V), dtype=np.float32)
    sc = default_scale(K) if scale is None else scale
    rc = lib.oracle_fused_recurrent_update_threads(
        B, T, H, HV, K, V, _p(q), _p(k), _p(v), _p(g), _p(beta), beta_per_v,
        ctypes.c_float(sc), int(use_qk_l2norm_in_kernel), _p(cu), N, sbf, _p(st),
        ctypes.c_int64(0 if st is None else st.shape[0]), _p(idx), _p(init), _p(final),
        _p(inter), ctypes.c_int64(0 if inter is None else inter.shape[1]), int(steps_per_token),
        _p(o), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_fused_recurrent_update failed: {rc}")
    return (bf16_round(o) if work_bf16 else o), (st if st is not None else final), inter


def snapshot_rollback(*, state, state_indices, intermediate_states, accepted):
    """Roll each request's state back to its snapshot after `accepted` draft
    tokens ("core.ssm.ops.gdp.fused_recurrent", intermediate_states).

    Returns the updated state copy."""
    lib = _load()
    st, bf = _state_copy(state)
    inter = np.ascontiguousarray(intermediate_states)
    if inter.dtype != st.dtype:
        raise TypeError("state and intermediate_states must share a dtype")
    idx = np.ascontiguousarray(state_indices, dtype=np.int32)
    acc = np.ascontiguousarray(accepted, dtype=np.int32)
    S, HV, K, V = st.shape
    rc = lib.oracle_snapshot_rollback(
        idx.shape[0], HV, K, V, st.itemsize, _p(st), ctypes.c_int64(S), _p(inter),
        ctypes.c_int64(inter.shape[1]), _p(idx), _p(acc))
    if rc != 0:
        raise ValueError(f"oracle_snapshot_rollback failed: {rc}")
    return st


def causal_conv1d(*, x, weight, slot_idx, row_offsets, bias=None, conv_state=None,
                  silu=False):
    """Pass-1 causal depthwise Conv1d producing qkv_conv_output (named on the
    "gated_delta_recurrence_fwd_gpu" page; the reading is stated in
    gdr_oracle.c).  x [T, C] float32 or uint16 (bf16 bits: the work dtype,
    whose output is rounded once); weight [C, W] and bias [C] float32;
    conv_state [slots, W-1, C] of x's dtype, or None (zero history, not
    updated), copied.  Returns (out [T, C] of x's dtype, conv_state_after)."""
    lib = _load()
    (xf,), bf = _work((x,))
    st = None
    if conv_state is not None:
        (st,), sbf = _work((conv_state,))
        if sbf != bf:
            raise TypeError("conv_state must have x's dtype")
        st = np.array(st, dtype=np.float32, order="C", copy=True)
    w = np.ascontiguousarray(weight, dtype=np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    off = np.ascontiguousarray(row_offsets, dtype=np.uint32)
    sl = np.ascontiguousarray(slot_idx, dtype=np.uint32)
    T, C = xf.shape
    W = w.shape[1]
    out = np.zeros((T, C), dtype=np.float32)
    rc = lib.oracle_causal_conv1d(
        sl.shape[0], C, W, _p(off), _p(sl), _p(xf), _p(w), _p(b), _p(st),
        ctypes.c_int64(0 if st is None else st.shape[0]), int(silu), _p(out))
    if rc != 0:
        raise ValueError(f"oracle_causal_conv1d failed: {rc}")
    if bf:
        return bf16_round(out), (None if st is None else bf16_round(st))
    return out, st


def fwd_output_shape(qkv_shape, state_shape):
    """Output shape of the forward ("gated_delta_recurrence_fwd_shape")."""
    return (int(qkv_shape[0]), int(state_shape[1]) * int(state_shape[3]))
