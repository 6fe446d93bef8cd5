"""The C ABI on the CPU: the library loads, exports every entry point that
include/gdr.h declares, and rejects bad arguments on the host before anything
is enqueued (no GPU needed: these calls never reach the HIP runtime)."""
import ctypes
import os
import re

import pytest

from gated_delta_rule_loop_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdr.h")

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH),
                                reason="libgdr.so not built (run __graft_entry__.build())")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\S.*?\b(gdr_\w+)\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("gdr_recurrence_fwd", "gdr_recurrence_verify_ring", "gdr_state_fold",
              "gdr_fused_recurrent_update", "gdr_snapshot_rollback", "gdr_causal_conv1d",
              "gdr_fwd_output_shape", "gdr_ring_record_elements", "gdr_last_error_message",
              "gdr_version"):
        assert n in names
    assert set(names) == set(B.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(B.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} declared in gdr.h but not exported"


def test_version_and_record_elements():
    assert "gfx950" in B.gdr_version()
    assert B.gdr_ring_record_elements(2, 128, 128) == 128 + 2 * 129
    assert B.gdr_ring_record_elements(0, 128, 128) == -1


FAKE = 0x10000  # never dereferenced: validation fails first


def T(shape, dtype=B.GDR_DTYPE_F32, stride=None, data=FAKE):
    d = B.GdrTensor()
    d.data = data
    d.dtype = dtype
    d.ndim = len(shape)
    if stride is None:
        stride, acc = [], 1
        for s in reversed(shape):
            stride.insert(0, acc)
            acc *= s
    for i, (s, st) in enumerate(zip(shape, stride)):
        d.shape[i] = s
        d.stride[i] = st
    return d


def fwd_args(B_=4, T_=10, nk=2, nv=4, K=16, **over):
    a = dict(out=T([T_, nv * K]), state=T([6, nv, K, K], B.GDR_DTYPE_BF16),
             slot=T([B_], B.GDR_DTYPE_U32), qkv=T([T_, 2 * nk * K + nv * K]),
             decay=T([T_, nv]), beta=T([T_, nv]), off=T([B_ + 1], B.GDR_DTYPE_U32))
    a.update(over)
    return a


def call_fwd(a, nv=4, nk=2):
    L = B.lib()
    r = lambda d: None if d is None else ctypes.byref(d)  # noqa: E731
    return L.gdr_recurrence_fwd(nv, nk, r(a["out"]), r(a["state"]), r(a["slot"]), r(a["qkv"]),
                                r(a["decay"]), r(a["beta"]), r(a["off"]), ctypes.c_float(-1),
                                1, None)


@pytest.mark.parametrize("case,code", [
    (dict(out=None), B.GDR_OK - 1),
    (dict(qkv=T([10, 63])), -1),                                  # wrong conv_dim
    (dict(decay=T([10, 3])), -1),                                 # wrong head count
    (dict(off=T([4], B.GDR_DTYPE_U32)), -1),                      # offsets must be B+1
    (dict(state=T([6, 4, 16, 16], B.GDR_DTYPE_U32)), -2),         # state dtype
    (dict(state=T([6, 4, 24, 24], B.GDR_DTYPE_BF16)), -2),        # head dim not built
    (dict(state=T([6, 4, 16, 32], B.GDR_DTYPE_BF16)), -2),        # K != V
    (dict(qkv=T([10, 128], stride=[256, 2])), -2),                  # innermost stride
    (dict(qkv=T([10, 128], data=FAKE + 4)), -2),                   # misaligned base
    (dict(state=T([6, 4, 16, 16], B.GDR_DTYPE_BF16, stride=[1024, 256, 17, 1])), -2),
    (dict(qkv=T([10, 128], B.GDR_DTYPE_BF16)), -2),               # work dtypes differ
    (dict(out=T([10, 64], B.GDR_DTYPE_BF16)), -2),                # output not the work dtype
    (dict(qkv=T([10, 128], B.GDR_DTYPE_BF16, stride=[132, 1]), decay=T([10, 4], B.GDR_DTYPE_BF16),
          beta=T([10, 4], B.GDR_DTYPE_BF16), out=T([10, 64], B.GDR_DTYPE_BF16)), -2),  # bf16 rows
])
def test_fwd_rejects_bad_arguments(case, code):
    rc = call_fwd(fwd_args(**case))
    assert rc == code
    assert B.gdr_last_error_message()


def test_fwd_rejects_bad_head_ratio():
    assert call_fwd(fwd_args(), nv=4, nk=3) == -1
    assert "multiple" in B.gdr_last_error_message()


def test_empty_batch_is_a_no_op():
    a = fwd_args(B_=0, T_=0)
    assert call_fwd(a) == 0
    assert B.gdr_last_error_message() == ""


def test_verify_requires_a_ring_with_room():
    L = B.lib()
    a = fwd_args()
    r = ctypes.byref
    small = T([8, 2, 4, 16 + 2 * 17 - 1])
    rc = L.gdr_recurrence_verify_ring(4, 2, r(a["out"]), r(a["state"]), r(a["slot"]),
                                      r(a["qkv"]), r(a["decay"]), r(a["beta"]), r(a["off"]),
                                      r(small), r(T([4], B.GDR_DTYPE_U32)), ctypes.c_float(-1), 1,
                                      None)
    assert rc == -1 and "record stride" in B.gdr_last_error_message()
    rc = L.gdr_recurrence_verify_ring(4, 2, r(a["out"]), r(a["state"]), r(a["slot"]),
                                      r(a["qkv"]), r(a["decay"]), r(a["beta"]), r(a["off"]),
                                      None, None, ctypes.c_float(-1), 1, None)
    assert rc == -1
    # a bf16 ring needs 16-byte outer strides (multiples of 8 elements)
    odd = T([8, 2, 4, 52], B.GDR_DTYPE_BF16)
    rc = L.gdr_recurrence_verify_ring(4, 2, r(a["out"]), r(a["state"]), r(a["slot"]),
                                      r(a["qkv"]), r(a["decay"]), r(a["beta"]), r(a["off"]),
                                      r(odd), r(T([4], B.GDR_DTYPE_U32)), ctypes.c_float(-1), 1,
                                      None)
    assert rc == -2 and "multiple of 8" in B.gdr_last_error_message()
    rc = L.gdr_state_fold(4, 2, r(a["state"]), r(a["slot"]), r(odd), r(T([4], B.GDR_DTYPE_U32)),
                          r(T([4], B.GDR_DTYPE_U32)), None)
    assert rc == -2


def test_fused_argument_checks():
    L = B.lib()
    r = lambda d: None if d is None else ctypes.byref(d)  # noqa: E731
    q = T([2, 3, 2, 16])
    v = T([2, 3, 4, 16])
    o = T([2, 3, 4, 16])

    def call(**kw):
        a = dict(q=q, k=q, v=v, g=None, beta=None, init=None, fin=None, cu=None, state=None,
                 idx=None, inter=None, spt=1, o=o)
        a.update(kw)
        return L.gdr_fused_recurrent_update(
            r(a["q"]), r(a["k"]), r(a["v"]), r(a["g"]), r(a["beta"]), ctypes.c_float(-1),
            r(a["init"]), r(a["fin"]), 1, r(a["cu"]), r(a["state"]), r(a["idx"]), r(a["inter"]),
            a["spt"], r(a["o"]), None)

    assert call(v=T([2, 3, 3, 16])) == -1                          # HV not a multiple of H
    assert call(cu=T([3], B.GDR_DTYPE_I32)) == -1                  # varlen needs B == 1
    assert call(spt=0) == -1
    assert call(inter=T([4, 3, 4, 16, 16], B.GDR_DTYPE_BF16)) == -1  # snapshots need a state
    assert call(beta=T([2, 3, 4, 8])) == -1                        # per-V beta must match v
    assert call(beta=T([2, 3, 4, 16], stride=[192, 64, 1, 4])) == -2  # V axis not unit stride
    assert call(v=T([2, 3, 4, 32]), o=T([2, 3, 4, 32])) == -2      # K != V
    assert call(v=T([2, 3, 4, 16], B.GDR_DTYPE_BF16)) == -2        # work dtypes differ
    st = T([5, 4, 16, 16], B.GDR_DTYPE_BF16)
    assert call(state=st, inter=T([5, 3, 4, 16, 16], B.GDR_DTYPE_F32)) == -2  # dtype mismatch
    assert call(state=st, idx=T([3], B.GDR_DTYPE_I32)) == -1       # indices must be [N]
    # q and k are read in aligned 4-element runs: their rows need 16-byte strides
    odd = T([2, 3, 2, 16], stride=[108, 36, 18, 1])
    assert call(q=odd) == -2 and "multiple of 4" in B.gdr_last_error_message()
    assert call(k=odd) == -2 and "multiple of 4" in B.gdr_last_error_message()
    assert call(q=T([2, 3, 2, 16], stride=[96, 32, 16, 2])) == -2  # innermost not unit


def test_output_shape_helper():
    L = B.lib()
    out = (ctypes.c_int64 * 2)()
    rc = L.gdr_fwd_output_shape(ctypes.byref(T([37, 8192])),
                                ctypes.byref(T([512, 32, 128, 128], B.GDR_DTYPE_BF16)), out)
    assert rc == 0 and (out[0], out[1]) == (37, 4096)


def test_rollback_argument_checks():
    L = B.lib()
    r = lambda d: None if d is None else ctypes.byref(d)  # noqa: E731
    st = T([6, 4, 16, 16], B.GDR_DTYPE_BF16)
    inter = T([6, 3, 4, 16, 16], B.GDR_DTYPE_BF16)
    idx = T([5], B.GDR_DTYPE_I32)
    acc = T([5], B.GDR_DTYPE_I32)
    assert L.gdr_snapshot_rollback(r(st), r(idx), r(T([6, 3, 4, 16, 16])), r(acc), None) == -2
    assert L.gdr_snapshot_rollback(r(st), r(idx), r(T([7, 3, 4, 16, 16], B.GDR_DTYPE_BF16)),
                                   r(acc), None) == -1
    assert L.gdr_snapshot_rollback(r(st), r(idx), r(inter), r(T([4], B.GDR_DTYPE_I32)),
                                   None) == -1
    assert L.gdr_snapshot_rollback(r(st), r(T([0], B.GDR_DTYPE_I32)), r(inter),
                                   r(T([0], B.GDR_DTYPE_I32)), None) == 0


def test_conv_argument_checks():
    L = B.lib()
    r = lambda d: None if d is None else ctypes.byref(d)  # noqa: E731

    def call(**kw):
        a = dict(out=T([10, 64], data=FAKE + 0x10000), x=T([10, 64]), w=T([64, 4]), b=None,
                 st=T([5, 3, 64]), slot=T([3], B.GDR_DTYPE_U32), off=T([4], B.GDR_DTYPE_U32),
                 flags=0)
        a.update(kw)
        return L.gdr_causal_conv1d(r(a["out"]), r(a["x"]), r(a["w"]), r(a["b"]), r(a["st"]),
                                   r(a["slot"]), r(a["off"]), a["flags"], None)

    assert call(w=T([64, 5])) == -2                               # width not built
    assert call(w=T([64, 1])) == -2
    assert call(x=T([10, 62]), out=T([10, 62], data=FAKE + 0x10000), w=T([62, 4]),
                st=T([5, 3, 62])) == -2                           # channels not 4-aligned
    assert call(out=T([10, 64], B.GDR_DTYPE_BF16, data=FAKE + 0x10000)) == -2  # work dtypes
    assert call(st=T([5, 2, 64])) == -1                           # history must be W-1
    assert call(st=T([5, 3, 64], B.GDR_DTYPE_BF16)) == -2         # history dtype
    assert call(slot=T([4], B.GDR_DTYPE_U32)) == -1               # slots must be [B]
    assert call(flags=4) == -1
    assert call(out=T([10, 64], data=FAKE + 0x1000), x=T([10, 64], data=FAKE + 0x1000)) == -1
    assert call(w=T([64, 4], stride=[1, 64])) == -2               # taps not unit stride
    assert call(x=T([0, 64]), out=T([0, 64], data=FAKE + 0x10000)) == 0  # no tokens: no-op
    # empty tensors as an allocator hands them over: null data, any strides
    assert call(x=T([0, 64], data=0, stride=[1, 7]), out=T([0, 64], data=0)) == 0
    assert call(x=T([10, 64], data=0)) == -1                      # a non-empty x must exist


def test_empty_tensors_may_have_null_data():
    """A zero-extent required tensor passes with a null pointer (no row to
    run: the calls return before any launch)."""
    a = fwd_args(B_=0, T_=0, slot=T([0], B.GDR_DTYPE_U32, data=0),
                 qkv=T([0, 128], data=0), out=T([0, 64], data=0), decay=T([0, 4], data=0),
                 beta=T([0, 4], data=0))
    assert call_fwd(a) == 0, B.gdr_last_error_message()
    a = fwd_args(slot=T([4], B.GDR_DTYPE_U32, data=0))          # 4 rows need slot_idx
    assert call_fwd(a) == -1


def test_fwd_rejects_a_grid_past_one_launch():
    """2^26 rows x 4 key heads of 16-token rows at K = V = 128, 8 value heads
    per key head: the long-row tiling would need 2^33 workgroups."""
    Bn, T_, nk, nv, K = 1 << 26, 1 << 30, 4, 32, 128
    a = dict(out=T([T_, nv * K]), state=T([6, nv, K, K], B.GDR_DTYPE_BF16),
             slot=T([Bn], B.GDR_DTYPE_U32), qkv=T([T_, 2 * nk * K + nv * K]),
             decay=T([T_, nv]), beta=T([T_, nv]), off=T([Bn + 1], B.GDR_DTYPE_U32))
    assert call_fwd(a, nv=nv, nk=nk) == -1
    assert "too large" in B.gdr_last_error_message()
