"""Randomised pins of the CPU oracle (CPU only): 40 seeded small shapes, each
checked against the independent float64 Householder form (tests/dense_ref.py)
and against the identities the verify page states (verify output == forward
output, float32-ring fold == forward over the prefix, long rows commit,
short rows leave the pool alone)."""
import numpy as np
import pytest

import oracle
from gated_delta_rule_loop_amd import workloads as wl
from tests import dense_ref
from tests import oracle_pins as P


def _case(i):
    r = np.random.Generator(np.random.PCG64(20000 + i))
    K, V = int(r.integers(1, 13)), int(r.integers(1, 11))
    nk = int(r.choice([1, 2, 3]))
    nv = nk * int(r.choice([1, 2, 3]))
    lengths = r.integers(0, 11, size=int(r.integers(1, 6)))
    scale = float(r.uniform(0.1, 1.0)) if r.random() < 0.5 else None
    return K, V, nk, nv, lengths, scale


@pytest.mark.parametrize("i", range(40))
def test_oracle_random_shapes(i):
    K, V, nk, nv, lengths, scale = _case(i)
    B = len(lengths)
    w = P.small_packed(21000 + i, lengths, nk=nk, nv=nv, K=K, V=V, slots=B + 2)
    kw = {} if scale is None else {"scale": scale}
    out, st = P.run_fwd(w, **kw)
    sc = oracle.default_scale(K) if scale is None else scale
    for b in range(B):
        for hv in range(nv):
            rr = P.row_head_inputs(w, b, hv)
            o_ref, S_ref = dense_ref.dense_walk(rr["S0"], rr["qs"], rr["ks"], rr["vs"], rr["a"],
                                                rr["beta"], sc, True)
            if rr["t1"] > rr["t0"]:
                P._close(out[rr["t0"]:rr["t1"], hv * V:(hv + 1) * V], o_ref, 1e-5,
                         f"case {i} o b{b} hv{hv}")
            P._close(st[w["slot_idx"][b], hv], S_ref, 1e-5, f"case {i} S b{b} hv{hv}")
    # verify / fold identities with a ring shorter than some rows
    ring_len = int(max(1, np.median(lengths)))
    ring = np.zeros((B + 1, nk, ring_len, oracle.ring_record_elements(nv // nk, K, V)),
                    np.float32)
    rsl = np.arange(B, dtype=np.uint32)[::-1].copy()
    args = {k: w[k] for k in ("qkv", "decay", "beta", "state", "slot_idx", "row_offsets",
                              "num_value_heads", "num_key_heads")}
    out_v, st_v, ring_v = oracle.recurrence_verify_ring(**args, ring=ring, ring_slot_idx=rsl,
                                                        **kw)
    assert np.array_equal(out_v.view(np.uint32), out.view(np.uint32)), "verify == forward"
    off = w["row_offsets"].astype(np.int64)
    for b, L in enumerate(lengths):
        s = w["slot_idx"][b]
        want = st[s] if L > ring_len else w["state"][s]
        assert np.array_equal(st_v[s], want), f"case {i} row {b} after verify"
    for n in range(0, int(lengths.max()) + 1):
        acc = np.array([min(n, L) if L <= ring_len else L for L in lengths], np.uint32)
        folded = oracle.state_fold(state=st_v, slot_idx=w["slot_idx"], ring=ring_v,
                                   ring_slot_idx=rsl, accepted=acc, num_value_heads=nv,
                                   num_key_heads=nk)
        keep = np.concatenate([np.arange(off[b], off[b] + acc[b]) for b in range(B)])
        offs = np.zeros(B + 1, np.uint32)
        offs[1:] = np.cumsum(acc)
        _, st_pre = P.run_fwd(dict(w, qkv=w["qkv"][keep], decay=w["decay"][keep],
                                   beta=w["beta"][keep], row_offsets=offs), **kw)
        sl = w["slot_idx"].astype(np.int64)
        assert np.array_equal(folded[sl].view(np.uint32), st_pre[sl].view(np.uint32)), (i, n)
