"""ctypes binding of libgdr.so (include/gdr.h).

Argument marshalling only: torch tensors on the HIP device are described as
gdr_tensor structs (data pointer, dtype, shape, strides in elements) and the
call is enqueued on torch's current stream.  Every step of the recurrence runs
in the library's kernels; there is no fallback of any kind - if the library is
missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdr.so")

GDR_OK = 0
GDR_DTYPE_F32, GDR_DTYPE_BF16, GDR_DTYPE_U32, GDR_DTYPE_I32 = 0, 1, 2, 3
GDR_FLAG_L2NORM_QK = 1
GDR_FLAG_CONV_SILU = 2
MAX_DIMS = 5

_DTYPES = {torch.float32: GDR_DTYPE_F32, torch.bfloat16: GDR_DTYPE_BF16,
           torch.int32: GDR_DTYPE_I32}
if hasattr(torch, "uint32"):
    _DTYPES[torch.uint32] = GDR_DTYPE_U32


class GdrTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * MAX_DIMS), ("stride", ctypes.c_int64 * MAX_DIMS)]


class GdrError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__(f"{fn} returned {code}: {msg}")
        self.code = code


_lib = None
EXPORTS = ("gdr_recurrence_fwd", "gdr_recurrence_verify_ring", "gdr_state_fold",
           "gdr_fused_recurrent_update", "gdr_snapshot_rollback", "gdr_causal_conv1d",
           "gdr_fwd_output_shape", "gdr_check_indices", "gdr_set_debug_checks",
           "gdr_ring_record_elements", "gdr_last_error_message", "gdr_version")


def lib():
    """Load libgdr.so (built by gated_delta_rule_loop_amd.build); raises if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m gated_delta_rule_loop_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(GdrTensor)
        i32, u32, f32, vp = ctypes.c_int32, ctypes.c_uint32, ctypes.c_float, ctypes.c_void_p
        L.gdr_recurrence_fwd.argtypes = [i32, i32, P, P, P, P, P, P, P, f32, u32, vp]
        L.gdr_recurrence_verify_ring.argtypes = [i32, i32, P, P, P, P, P, P, P, P, P, f32, u32, vp]
        L.gdr_state_fold.argtypes = [i32, i32, P, P, P, P, P, vp]
        L.gdr_fused_recurrent_update.argtypes = [P, P, P, P, P, f32, P, P, u32, P, P, P, P, i32,
                                                 P, vp]
        L.gdr_snapshot_rollback.argtypes = [P, P, P, P, vp]
        L.gdr_causal_conv1d.argtypes = [P, P, P, P, P, P, P, u32, vp]
        L.gdr_fwd_output_shape.argtypes = [P, P, ctypes.POINTER(ctypes.c_int64)]
        i64 = ctypes.c_int64
        L.gdr_check_indices.argtypes = [i64, vp, i64, vp, i64, vp, i64, i64, vp]
        L.gdr_set_debug_checks.argtypes = [ctypes.c_int]
        L.gdr_ring_record_elements.argtypes = [i32, i32, i32]
        L.gdr_ring_record_elements.restype = ctypes.c_int64
        L.gdr_last_error_message.restype = ctypes.c_char_p
        L.gdr_version.restype = ctypes.c_char_p
        for name in EXPORTS[:9]:
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def describe(t, *, allow_host=False):
    """gdr_tensor for a torch tensor (None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"expected a torch.Tensor, got {type(t)}")
    if not allow_host and not t.is_cuda:
        raise ValueError("gdr kernels take device tensors")
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}")
    if t.dim() > MAX_DIMS:
        raise ValueError("rank above 5")
    d = GdrTensor()
    d.data = t.data_ptr() if t.numel() > 0 else (t.data_ptr() or None)
    d.dtype = _DTYPES[t.dtype]
    d.ndim = t.dim()
    for i, (s, st) in enumerate(zip(t.shape, t.stride())):
        d.shape[i] = s
        d.stride[i] = st
    return d


def _ref(d):
    return None if d is None else ctypes.byref(d)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn, rc):
    if rc != GDR_OK:
        raise GdrError(fn, rc, lib().gdr_last_error_message().decode())


def _scale(scale):
    return ctypes.c_float(-1.0 if scale is None or (isinstance(scale, float) and math.isnan(scale))
                          else float(scale))


def gdr_recurrence_fwd(recurrence_output, recurrent_state, slot_idx, qkv_conv_output,
                       decay_per_token, beta_per_token, input_row_offsets, *,
                       num_value_heads, num_key_heads, scale=None, l2norm=True, stream=None):
    """Slot-indexed ragged forward (page "gated_delta_recurrence_fwd_gpu").
    Writes recurrence_output and updates recurrent_state in place."""
    ds = [describe(x) for x in (recurrence_output, recurrent_state, slot_idx, qkv_conv_output,
                                decay_per_token, beta_per_token, input_row_offsets)]
    rc = lib().gdr_recurrence_fwd(num_value_heads, num_key_heads, *[_ref(d) for d in ds],
                                  _scale(scale), GDR_FLAG_L2NORM_QK if l2norm else 0,
                                  _stream(stream))
    _check("gdr_recurrence_fwd", rc)
    return recurrence_output


def gdr_recurrence_verify_ring(recurrence_output, recurrent_state, slot_idx, qkv_conv_output,
                               decay_per_token, beta_per_token, input_row_offsets, ring,
                               ring_slot_idx, *, num_value_heads, num_key_heads, scale=None,
                               l2norm=True, stream=None):
    """Verify window recording the ring (page "gated_delta_recurrence_verify_ring_gpu")."""
    ds = [describe(x) for x in (recurrence_output, recurrent_state, slot_idx, qkv_conv_output,
                                decay_per_token, beta_per_token, input_row_offsets, ring,
                                ring_slot_idx)]
    rc = lib().gdr_recurrence_verify_ring(num_value_heads, num_key_heads,
                                          *[_ref(d) for d in ds], _scale(scale),
                                          GDR_FLAG_L2NORM_QK if l2norm else 0, _stream(stream))
    _check("gdr_recurrence_verify_ring", rc)
    return recurrence_output


def gdr_state_fold(recurrent_state, slot_idx, ring, ring_slot_idx, accepted, *,
                   num_value_heads, num_key_heads, stream=None):
    """Fold accepted ring records into the live state."""
    ds = [describe(x) for x in (recurrent_state, slot_idx, ring, ring_slot_idx, accepted)]
    rc = lib().gdr_state_fold(num_value_heads, num_key_heads, *[_ref(d) for d in ds],
                              _stream(stream))
    _check("gdr_state_fold", rc)
    return recurrent_state


def gdr_fused_recurrent_update(q, k, v, g=None, beta=None, scale=None, initial_state=None,
                               output_final_state=False, use_qk_l2norm_in_kernel=False,
                               cu_seqlens=None, state=None, state_indices=None,
                               intermediate_states=None, steps_per_token=1, *, o=None,
                               final_state=None, stream=None):
    """Fused recurrent update (page "core.ssm.ops.gdp.fused_recurrent").

    Returns (o, final_state): final_state is `state` itself when a cache is
    given, the dense final state when output_final_state, else None.  o (of
    v's dtype) and a dense final state are allocated here with torch when not
    passed in."""
    if o is None:
        o = torch.empty(v.shape, dtype=v.dtype, device=v.device)
    if state is None and output_final_state and final_state is None:
        N = q.shape[0] if cu_seqlens is None else cu_seqlens.shape[0] - 1
        dt = initial_state.dtype if initial_state is not None else torch.float32
        final_state = torch.empty((N, v.shape[2], q.shape[3], v.shape[3]), dtype=dt,
                                  device=v.device)
    args = [describe(x) for x in (q, k, v, g, beta)]
    init_d, fin_d = describe(initial_state), describe(final_state)
    rest = [describe(x) for x in (cu_seqlens, state, state_indices, intermediate_states)]
    flags = GDR_FLAG_L2NORM_QK if use_qk_l2norm_in_kernel else 0
    rc = lib().gdr_fused_recurrent_update(*[_ref(d) for d in args], _scale(scale), _ref(init_d),
                                          _ref(fin_d), flags, *[_ref(d) for d in rest],
                                          int(steps_per_token), _ref(describe(o)),
                                          _stream(stream))
    _check("gdr_fused_recurrent_update", rc)
    return o, (state if state is not None else final_state)


def gdr_snapshot_rollback(state, state_indices, intermediate_states, accepted, *,
                          stream=None):
    """Roll each request's state back to its snapshot after `accepted` draft
    tokens (page "core.ssm.ops.gdp.fused_recurrent", intermediate_states)."""
    ds = [describe(x) for x in (state, state_indices, intermediate_states, accepted)]
    rc = lib().gdr_snapshot_rollback(*[_ref(d) for d in ds], _stream(stream))
    _check("gdr_snapshot_rollback", rc)
    return state


def gdr_causal_conv1d(x, weight, input_row_offsets, *, bias=None, conv_state=None,
                      slot_idx=None, silu=False, out=None, stream=None):
    """Pass-1 causal depthwise Conv1d producing qkv_conv_output (page
    "gated_delta_recurrence_fwd_gpu", Args).  Returns out (allocated here with
    torch, x's dtype and shape, when not passed in); conv_state is updated in
    place."""
    if out is None:
        out = torch.empty(x.shape, dtype=x.dtype, device=x.device)
    ds = [describe(t) for t in (out, x, weight, bias, conv_state, slot_idx, input_row_offsets)]
    rc = lib().gdr_causal_conv1d(*[_ref(d) for d in ds], GDR_FLAG_CONV_SILU if silu else 0,
                                 _stream(stream))
    _check("gdr_causal_conv1d", rc)
    return out


def gdr_fwd_output_shape(qkv_conv_output, recurrent_state):
    """Output shape of the forward (page "gated_delta_recurrence_fwd_shape")."""
    out = (ctypes.c_int64 * 2)()
    rc = lib().gdr_fwd_output_shape(_ref(describe(qkv_conv_output, allow_host=True)),
                                    _ref(describe(recurrent_state, allow_host=True)), out)
    _check("gdr_fwd_output_shape", rc)
    return (out[0], out[1])


def gdr_check_indices(rows, *, row_offsets=None, total_tokens=0, slots=None, num_slots=0,
                      ring_idx=None, ring_rows=0, ring_len=0, accepted=None):
    """Host-side index check (host arrays: NumPy or CPU tensors of 32-bit
    integers; -1 / 0xFFFFFFFF is padding).  Raises GdrError on a violation."""
    import numpy as np  # noqa: PLC0415
    keep = []

    def ptr(a):
        if a is None:
            return None
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().numpy()
        a = np.ascontiguousarray(a)
        if a.dtype.itemsize != 4 or a.dtype.kind not in "iu":
            raise TypeError("index arrays must hold 32-bit integers")
        keep.append(a)
        return a.ctypes.data_as(ctypes.c_void_p)

    rc = lib().gdr_check_indices(int(rows), ptr(row_offsets), int(total_tokens), ptr(slots),
                                 int(num_slots), ptr(ring_idx), int(ring_rows), int(ring_len),
                                 ptr(accepted))
    _check("gdr_check_indices", rc)


def gdr_set_debug_checks(enable):
    """Turn the per-call index checks on or off; returns the previous setting."""
    return bool(lib().gdr_set_debug_checks(1 if enable else 0))


def gdr_ring_record_elements(group, key_head_dim, value_head_dim):
    return int(lib().gdr_ring_record_elements(group, key_head_dim, value_head_dim))


def gdr_version():
    return lib().gdr_version().decode()


def gdr_last_error_message():
    return lib().gdr_last_error_message().decode()
