"""Pins that tie the CPU oracle to facts other than itself.

Each pin_* function raises AssertionError when the oracle currently routed
through the oracle package disagrees with what the pages or the mathematics
fix.  test_oracle_pins.py runs them against the real oracle;
test_oracle_mutations.py runs them against builds with planted mistakes and
expects some pin to fail for each.
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch

import oracle
from gated_delta_rule_loop_amd import workloads as wl
from tests import dense_ref

HERE = os.path.dirname(os.path.abspath(__file__))


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def state_f32(st):
    return wl.bf16_bits_to_f32(st) if st.dtype == np.uint16 else np.asarray(st, np.float32)


def row_head_inputs(w, b, hv):
    """Slices of a packed workload for row b, value head hv (no arithmetic)."""
    nk, nv = w["num_key_heads"], w["num_value_heads"]
    G = nv // nk
    h = hv // G
    st = w["state"]
    K, V = st.shape[2], st.shape[3]
    t0, t1 = int(w["row_offsets"][b]), int(w["row_offsets"][b + 1])
    x = w["qkv"][t0:t1]
    qs = x[:, h * K:(h + 1) * K]
    ks = x[:, nk * K + h * K:nk * K + (h + 1) * K]
    vs = x[:, 2 * nk * K + hv * V:2 * nk * K + (hv + 1) * V]
    return dict(t0=t0, t1=t1, qs=qs, ks=ks, vs=vs, a=w["decay"][t0:t1, hv],
                beta=w["beta"][t0:t1, hv], S0=state_f32(st)[w["slot_idx"][b], hv])


def small_packed(seed, lengths, nk=2, nv=4, K=8, V=4, slots=7, state_dtype="f32", sigma=0.3):
    w = wl.packed_inputs(_rng(seed), lengths, nk=nk, nv=nv, K=K, V=V, slots=slots,
                         state_dtype=state_dtype, state_sigma=sigma)
    return w


def run_fwd(w, **kw):
    args = {k: w[k] for k in ("qkv", "decay", "beta", "state", "slot_idx", "row_offsets",
                              "num_value_heads", "num_key_heads")}
    args.update(kw)
    if "scale" in w and "scale" not in kw:
        args["scale"] = w["scale"]
    return oracle.recurrence_fwd(**args)


def _close(got, want, rel, what):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    scale = max(np.abs(want).max(initial=0.0), 1e-30)
    err = np.abs(got - want).max(initial=0.0)
    assert err <= rel * scale, f"{what}: max err {err:.3e} > {rel:.1e} * {scale:.3e}"


# ------------------------------------------------------------------ pins ---

def pin_dense_fp64():
    """Elementwise fp32 oracle == fp64 Householder matrix form (K != V, GQA,
    ragged with an empty row, L2 norm on, non-default scale)."""
    w = small_packed(11, [0, 5, 9, 1], K=8, V=4)
    scale = 0.37
    out, st = run_fwd(w, scale=scale, l2norm=True)
    S_all = state_f32(st)
    for b in range(4):
        for hv in range(4):
            r = row_head_inputs(w, b, hv)
            o_ref, S_ref = dense_ref.dense_walk(r["S0"], r["qs"], r["ks"], r["vs"], r["a"],
                                                r["beta"], scale, True)
            if r["t1"] > r["t0"]:
                _close(out[r["t0"]:r["t1"], hv * 4:(hv + 1) * 4], o_ref, 1e-5, f"o b{b} hv{hv}")
            _close(S_all[w["slot_idx"][b], hv], S_ref, 1e-5, f"S b{b} hv{hv}")


def pin_dense_unrolled():
    """The fp64 step-by-step form == the unrolled product closed form."""
    rng = _rng(12)
    K, V, T = 6, 5, 7
    S0 = rng.standard_normal((K, V))
    ks, vs, qs = rng.standard_normal((T, K)), rng.standard_normal((T, V)), rng.standard_normal((T, K))
    a, beta = rng.uniform(0.2, 1, T), rng.uniform(0, 1, T)
    _, S = dense_ref.dense_walk(S0, qs, ks, vs, a, beta, 1.0, True)
    S2 = dense_ref.unrolled_state(S0, ks, vs, a, beta, True)
    _close(S, S2, 1e-12, "unrolled")


def pin_beta_zero_decay_only():
    """beta = 0: S_T = (prod a) S_0 and o_t = scale (prod_{s<=t} a_s) S_0^T q_hat_t."""
    w = small_packed(13, [4, 7], K=8, V=8)
    w["beta"][:] = 0.0
    out, st = run_fwd(w, scale=0.5)
    for b in range(2):
        for hv in range(4):
            r = row_head_inputs(w, b, hv)
            cum = np.cumprod(r["a"].astype(np.float64))
            S0 = r["S0"].astype(np.float64)
            qh = np.array([dense_ref.l2n(q) for q in r["qs"]])
            o_ref = 0.5 * cum[:, None] * (qh @ S0)
            _close(out[r["t0"]:r["t1"], hv * 8:(hv + 1) * 8], o_ref, 1e-5, "o beta=0")
            _close(state_f32(st)[w["slot_idx"][b], hv], cum[-1] * S0, 1e-5, "S beta=0")


def pin_delta_retrieval():
    """One step with unit-norm k: S'^T k = (1 - beta) a S^T k + beta v; with a = 1
    and beta = 1 the write makes the state return exactly v for k."""
    for a_one in (True, False):
        w = small_packed(14 + a_one, [1, 1, 1], K=16, V=8)
        if a_one:
            w["decay"][:] = 1.0
            w["beta"][:] = 1.0
        out, st = run_fwd(w)
        for b in range(3):
            for hv in range(4):
                r = row_head_inputs(w, b, hv)
                k = dense_ref.l2n(r["ks"][0])
                S1 = state_f32(st)[w["slot_idx"][b], hv].astype(np.float64)
                a, be = float(r["a"][0]), float(r["beta"][0])
                want = (1 - be) * a * (r["S0"].astype(np.float64).T @ k) + be * r["vs"][0]
                _close(S1.T @ k, want, 2e-5, "retrieval after write")


def pin_scalar_state():
    """K = V = 1 with the norm on: k_hat = sign(k), so
    s' = a (1 - beta) s + beta sign(k) v and o = scale sign(q) s'."""
    rng = _rng(16)
    T = 6
    w = small_packed(16, [T], nk=1, nv=1, K=1, V=1, slots=2)
    # keep |q|, |k| away from 0 so that eps is negligible
    w["qkv"][:, :2] = np.sign(w["qkv"][:, :2]) * rng.uniform(0.5, 2.0, (T, 2))
    out, st = run_fwd(w, scale=0.8)
    s = float(state_f32(w["state"])[w["slot_idx"][0], 0, 0, 0])
    for t in range(T):
        q, k, v = w["qkv"][t]
        a, be = float(w["decay"][t, 0]), float(w["beta"][t, 0])
        s = a * (1 - be) * s + be * np.sign(k) * v
        assert abs(out[t, 0] - 0.8 * np.sign(q) * s) <= 1e-5 * max(1.0, abs(s)), (t, out[t, 0], s)
    assert abs(state_f32(st)[w["slot_idx"][0], 0, 0, 0] - s) <= 1e-5 * max(1.0, abs(s))


def pin_gather_probe(state_dtype="bf16"):
    """a = 1, beta = 0, no norm, scale 1, one-hot q_t at i*(t, key head):
    o[t, hv] is exactly row i* of that row's slot state (indexing of offsets,
    slots, GQA key head and the S^T q orientation), and no slot changes."""
    rng = _rng(17)
    nk, nv, K, V = 2, 6, 8, 4
    w = small_packed(17, [3, 0, 5, 2], nk=nk, nv=nv, K=K, V=V, slots=9, state_dtype=state_dtype)
    T = w["qkv"].shape[0]
    w["decay"][:] = 1.0
    w["beta"][:] = 0.0
    istar = rng.integers(0, K, size=(T, nk))
    w["qkv"][:, :nk * K] = 0.0
    for t in range(T):
        for h in range(nk):
            w["qkv"][t, h * K + istar[t, h]] = 1.0
    out, st = run_fwd(w, scale=1.0, l2norm=False)
    S0 = state_f32(w["state"])
    G = nv // nk
    for b in range(4):
        t0, t1 = w["row_offsets"][b], w["row_offsets"][b + 1]
        for t in range(t0, t1):
            for hv in range(nv):
                want = S0[w["slot_idx"][b], hv, istar[t, hv // G], :]
                assert np.array_equal(out[t, hv * V:(hv + 1) * V], want), (b, t, hv)
    assert np.array_equal(np.asarray(st).view(np.uint8), np.asarray(w["state"]).view(np.uint8))


def pin_scatter_probe():
    """a = 0, beta = 1, no norm, one-hot k_t = e_i* on the last token: the
    stored state of the row is exactly e_i* v^T (v rounded to bf16 first so the
    bf16 store is exact); slots not in the batch are bit-unchanged."""
    rng = _rng(18)
    nk, nv, K, V = 2, 4, 8, 8
    w = small_packed(18, [2, 4, 1], nk=nk, nv=nv, K=K, V=V, slots=8, state_dtype="bf16")
    T = w["qkv"].shape[0]
    w["decay"][:] = 0.0
    w["beta"][:] = 1.0
    vpart = w["qkv"][:, 2 * nk * K:]
    w["qkv"][:, 2 * nk * K:] = wl.bf16_bits_to_f32(wl.to_bf16_bits(vpart))
    istar = rng.integers(0, K, size=(T, nk))
    w["qkv"][:, nk * K:2 * nk * K] = 0.0
    for t in range(T):
        for h in range(nk):
            w["qkv"][t, nk * K + h * K + istar[t, h]] = 1.0
    _, st = run_fwd(w, scale=1.0, l2norm=False)
    S1 = state_f32(st)
    G = nv // nk
    for b in range(3):
        tl = int(w["row_offsets"][b + 1]) - 1
        for hv in range(nv):
            want = np.zeros((K, V), np.float32)
            want[istar[tl, hv // G]] = w["qkv"][tl, 2 * nk * K + hv * V:2 * nk * K + (hv + 1) * V]
            assert np.array_equal(S1[w["slot_idx"][b], hv], want), (b, hv)
    others = np.setdiff1d(np.arange(8), w["slot_idx"])
    assert np.array_equal(st[others], w["state"][others])


def pin_linearity_pow2():
    """Scaling v and S_0 by 2 scales every output and stored state by exactly 2
    (the recurrence is linear in them and doubling commutes with rounding)."""
    w = small_packed(19, [3, 6], K=8, V=8, state_dtype="bf16")
    out1, st1 = run_fwd(w)
    w2 = dict(w)
    w2["qkv"] = w["qkv"].copy()
    w2["qkv"][:, 2 * 2 * 8:] *= 2.0
    w2["state"] = wl.to_bf16_bits(2.0 * state_f32(w["state"]))
    out2, st2 = run_fwd(w2)
    assert np.array_equal(out2, 2.0 * out1)
    assert np.array_equal(state_f32(st2), 2.0 * state_f32(st1))


def pin_verify_fold_identities():
    """Verify page: verify output == forward output; verify leaves the state of
    rows that fit the ring untouched; a longer row commits like the forward and
    records nothing; with a float32 ring, folding n accepted tokens equals the
    forward over the first n tokens bit for bit, for every n; n = 0 and
    n > ring_len leave the state alone."""
    ring_len = 4
    lengths = [1, 4, 6, 3, 2, 5]
    nk, nv, K, V = 2, 4, 8, 8
    w = small_packed(20, lengths, nk=nk, nv=nv, K=K, V=V, slots=10, state_dtype="bf16")
    G = nv // nk
    stride = wl.ring_record_stride(G, K, V, align=8)
    rng = _rng(21)
    ring = np.zeros((7, nk, ring_len, stride), np.float32)
    rslot = rng.choice(7, size=len(lengths), replace=False).astype(np.uint32)
    base = {k: w[k] for k in ("qkv", "decay", "beta", "state", "slot_idx", "row_offsets",
                              "num_value_heads", "num_key_heads")}
    out_f, st_f = oracle.recurrence_fwd(**base)
    out_v, st_v, ring_v = oracle.recurrence_verify_ring(**base, ring=ring, ring_slot_idx=rslot)
    assert np.array_equal(out_v, out_f)
    for b, L in enumerate(lengths):
        s = w["slot_idx"][b]
        if L <= ring_len:
            assert np.array_equal(st_v[s], w["state"][s])
        else:
            assert np.array_equal(st_v[s], st_f[s])
            assert not ring_v[rslot[b]].any()
    for n in range(0, max(lengths) + 1):
        acc = np.array([min(n, L) if L <= ring_len else L for L in lengths], np.uint32)
        folded = oracle.state_fold(state=st_v, slot_idx=w["slot_idx"], ring=ring_v,
                                   ring_slot_idx=rslot, accepted=acc, num_value_heads=nv,
                                   num_key_heads=nk)
        # forward over the accepted prefix of each row
        pre_len = [int(a) for a in acc]
        keep = np.concatenate([np.arange(w["row_offsets"][b], w["row_offsets"][b] + pre_len[b])
                               for b in range(len(lengths))]).astype(np.int64)
        offs = np.zeros(len(lengths) + 1, np.uint32)
        offs[1:] = np.cumsum(pre_len)
        pre = dict(base, qkv=w["qkv"][keep], decay=w["decay"][keep], beta=w["beta"][keep],
                   row_offsets=offs)
        _, st_pre = oracle.recurrence_fwd(**pre)
        for b, L in enumerate(lengths):
            s = w["slot_idx"][b]
            if L <= ring_len:
                assert np.array_equal(folded[s], st_pre[s]), (n, b)
            else:  # count above ring_len: the fold skips the row
                assert np.array_equal(folded[s], st_v[s]), (n, b)


def pin_replicated_heads():
    """GQA: nv/nk value heads share key head hv // (nv/nk).  Giving every value
    head its own copy of that key head's q and k must change nothing."""
    nk, nv, K, V = 2, 4, 8, 4
    w = small_packed(22, [3, 5], nk=nk, nv=nv, K=K, V=V, slots=4, state_dtype="bf16")
    out1, st1 = run_fwd(w)
    x = w["qkv"]
    q = x[:, :nk * K].reshape(-1, nk, K)
    k = x[:, nk * K:2 * nk * K].reshape(-1, nk, K)
    rep = np.arange(nv) // (nv // nk)
    x2 = np.concatenate([q[:, rep].reshape(len(x), -1), k[:, rep].reshape(len(x), -1),
                         x[:, 2 * nk * K:]], axis=1)
    w2 = dict(w, qkv=np.ascontiguousarray(x2), num_key_heads=nv)
    out2, st2 = run_fwd(w2)
    assert np.array_equal(out1, out2)
    assert np.array_equal(st1, st2)


def pin_fused_matches_packed():
    """The fused update's [B, T, H, K] layout with g = None (a = 1), cu_seqlens
    (varlen) and a pool computes the same walk as the packed forward with
    decay = 1; dense initial/final states equal the pool path; padding rows
    give zero output and touch nothing."""
    nk, nv, K, V = 2, 4, 8, 8
    lengths = [3, 5, 2]
    w = small_packed(23, lengths, nk=nk, nv=nv, K=K, V=V, slots=6, state_dtype="bf16")
    w["decay"][:] = 1.0
    out_p, st_p = run_fwd(w)
    T = w["qkv"].shape[0]
    x = w["qkv"]
    q = x[:, :nk * K].reshape(1, T, nk, K)
    k = x[:, nk * K:2 * nk * K].reshape(1, T, nk, K)
    v = x[:, 2 * nk * K:].reshape(1, T, nv, V)
    beta = w["beta"].reshape(1, T, nv)
    cu = w["row_offsets"].astype(np.int32)
    o, st, _ = oracle.fused_recurrent_update(
        q=q, k=k, v=v, beta=beta, use_qk_l2norm_in_kernel=True, cu_seqlens=cu,
        state=w["state"], state_indices=w["slot_idx"].astype(np.int32))
    assert np.array_equal(o.reshape(T, nv * V), out_p)
    assert np.array_equal(st, st_p)
    # dense initial / final state path, row by row (equal lengths needed: use row 0)
    L0 = lengths[0]
    init = w["state"][w["slot_idx"][:1]]
    o2, fin, _ = oracle.fused_recurrent_update(
        q=q[:, :L0], k=k[:, :L0], v=v[:, :L0], beta=beta[:, :L0], initial_state=init,
        output_final_state=True, use_qk_l2norm_in_kernel=True)
    assert np.array_equal(o2.reshape(L0, nv * V), out_p[:L0])
    assert np.array_equal(fin[0], st_p[w["slot_idx"][0]])
    # padding row: zero output, nothing touched
    idx = w["slot_idx"].astype(np.int32).copy()
    idx[1] = -1
    o3, st3, _ = oracle.fused_recurrent_update(
        q=q, k=k, v=v, beta=beta, use_qk_l2norm_in_kernel=True, cu_seqlens=cu,
        state=w["state"], state_indices=idx)
    t0, t1 = cu[1], cu[2]
    assert np.array_equal(o3[0, t0:t1], np.zeros_like(o3[0, t0:t1]))
    assert not np.signbit(o3[0, t0:t1]).any()
    assert np.array_equal(st3[w["slot_idx"][1]], w["state"][w["slot_idx"][1]])


def pin_snapshots():
    """intermediate[slot, i] is the state after draft token i, i.e. the state a
    run over the first (i+1) * steps_per_token steps stores; padding rows write
    no snapshot; the last snapshot equals the final state."""
    rng = _rng(24)
    w = wl.gdp_inputs(rng, B=5, S_draft=3, M=2, H=2, HV=4, K=8, V=8, slots=9, pad_frac=0.2,
                      state_sigma=0.2)
    args = {k: w[k] for k in ("q", "k", "v", "g", "beta", "state", "state_indices",
                              "intermediate_states", "steps_per_token",
                              "use_qk_l2norm_in_kernel", "scale")}
    o, st, inter = oracle.fused_recurrent_update(**args)
    M = w["steps_per_token"]
    for i in range(3):
        n_steps = (i + 1) * M
        sub = dict(args, q=w["q"][:, :n_steps], k=w["k"][:, :n_steps], v=w["v"][:, :n_steps],
                   g=w["g"][:, :n_steps], beta=w["beta"][:, :n_steps], intermediate_states=None)
        _, st_i, _ = oracle.fused_recurrent_update(**sub)
        for b, idx in enumerate(w["state_indices"]):
            if idx < 0:
                continue
            assert np.array_equal(inter[idx, i], st_i[idx]), (i, b)
    for b, idx in enumerate(w["state_indices"]):
        if idx < 0:
            assert not o[b].any()
        else:
            assert np.array_equal(inter[idx, -1], st[idx])
    touched = set(int(x) for x in w["state_indices"] if x >= 0)
    for s in range(9):
        if s not in touched:
            assert np.array_equal(inter[s], w["intermediate_states"][s])
            assert np.array_equal(st[s], w["state"][s])


def pin_snapshot_rollback():
    """Rolling a request back to its snapshot after n accepted draft tokens
    gives the state a run over the first n * steps_per_token steps stores;
    n = 0, n past the buffer and padding requests leave the state alone."""
    rng = _rng(26)
    w = wl.gdp_inputs(rng, B=6, S_draft=3, M=2, H=2, HV=4, K=8, V=8, slots=9, pad_frac=0.2,
                      state_sigma=0.2)
    args = {k: w[k] for k in ("q", "k", "v", "g", "beta", "state", "state_indices",
                              "intermediate_states", "steps_per_token",
                              "use_qk_l2norm_in_kernel", "scale")}
    _, st, inter = oracle.fused_recurrent_update(**args)
    M = w["steps_per_token"]
    idx = w["state_indices"]
    acc = np.full(len(idx), 2, np.int32)
    active = np.flatnonzero(idx >= 0)
    acc[active] = np.resize(np.array([1, 2, 3, 0, 4], np.int32), len(active))
    rolled = oracle.snapshot_rollback(state=st, state_indices=idx, intermediate_states=inter,
                                      accepted=acc)
    for b, i in enumerate(idx):
        if i < 0:
            continue
        n = int(acc[b])
        if 1 <= n <= 3:
            sub = dict(args, q=w["q"][:, :n * M], k=w["k"][:, :n * M], v=w["v"][:, :n * M],
                       g=w["g"][:, :n * M], beta=w["beta"][:, :n * M], intermediate_states=None)
            _, st_n, _ = oracle.fused_recurrent_update(**sub)
            assert np.array_equal(rolled[i], st_n[i]), (b, n)
        else:
            assert np.array_equal(rolled[i], st[i]), (b, n)
    others = np.setdiff1d(np.arange(9), idx[idx >= 0])
    assert np.array_equal(rolled[others], st[others])


def pin_per_v_beta():
    """Fused-update page, beta of shape [B, T, HV, V]: each value column j has
    its own transition a (I - beta_j k k^T), checked against the fp64 matrix
    form column by column; a per-column beta whose columns are all equal is
    the head-wise beta, bit for bit."""
    rng = _rng(27)
    w = wl.gdp_inputs(rng, B=3, S_draft=3, M=2, H=2, HV=4, K=8, V=6, slots=5, pad_frac=0.0,
                      state_sigma=0.3, state_dtype="f32", beta_per_v=True)
    args = {k: w[k] for k in ("q", "k", "v", "g", "beta", "state", "state_indices",
                              "use_qk_l2norm_in_kernel", "scale")}
    o, st, _ = oracle.fused_recurrent_update(**args)
    G = 4 // 2
    for b, idx in enumerate(w["state_indices"]):
        for hv in range(4):
            h = hv // G
            o_ref, S_ref = dense_ref.dense_walk(
                w["state"][idx, hv], w["q"][b, :, h], w["k"][b, :, h], w["v"][b, :, hv],
                np.exp(w["g"][b, :, hv].astype(np.float64)), w["beta"][b, :, hv], w["scale"],
                True)
            _close(o[b, :, hv], o_ref, 1e-5, f"o b{b} hv{hv}")
            _close(st[idx, hv], S_ref, 1e-5, f"S b{b} hv{hv}")
    head = w["beta"][..., 0]
    flat = np.ascontiguousarray(np.repeat(head[..., None], 6, axis=-1))
    o1, st1, _ = oracle.fused_recurrent_update(**dict(args, beta=head))
    o2, st2, _ = oracle.fused_recurrent_update(**dict(args, beta=flat))
    assert np.array_equal(o1, o2)
    assert np.array_equal(st1, st2)


def pin_bf16_ring():
    """Verify page, ring_dtype bfloat16: every ring element is the float32
    record rounded to bf16 once; folding a bf16 ring equals folding a float32
    ring that holds the widened values, bit for bit; and it lands within the
    bf16 rounding of the records from the forward over the accepted prefix."""
    ring_len = 4
    lengths = [2, 4, 3, 6]
    nk, nv, K, V = 2, 4, 8, 8
    w = small_packed(28, lengths, nk=nk, nv=nv, K=K, V=V, slots=6, state_dtype="f32")
    stride = wl.ring_record_stride(nv // nk, K, V, align=8)
    rslot = np.array([3, 0, 2, 1], np.uint32)
    base = {k: w[k] for k in ("qkv", "decay", "beta", "state", "slot_idx", "row_offsets",
                              "num_value_heads", "num_key_heads")}
    ring_f = np.zeros((4, nk, ring_len, stride), np.float32)
    ring_b = np.zeros((4, nk, ring_len, stride), np.uint16)
    out_f, st_f, rf = oracle.recurrence_verify_ring(**base, ring=ring_f, ring_slot_idx=rslot)
    out_b, st_b, rb = oracle.recurrence_verify_ring(**base, ring=ring_b, ring_slot_idx=rslot)
    assert np.array_equal(out_f, out_b)
    assert np.array_equal(st_f, st_b)
    assert np.array_equal(rb, oracle.bf16_round(rf))
    acc = np.array([1, 4, 3, 6], np.uint32)
    fold = dict(slot_idx=w["slot_idx"], ring_slot_idx=rslot, accepted=acc, num_value_heads=nv,
                num_key_heads=nk)
    s_b = oracle.state_fold(state=st_b, ring=rb, **fold)
    s_w = oracle.state_fold(state=st_b, ring=np.ascontiguousarray(wl.bf16_bits_to_f32(rb)),
                            **fold)
    assert np.array_equal(s_b, s_w)
    s_f = oracle.state_fold(state=st_f, ring=rf, **fold)
    for b in range(3):
        s = w["slot_idx"][b]
        _close(s_b[s], s_f[s], 2e-2, f"bf16 ring fold row {b}")
        assert not np.array_equal(s_b[s], s_f[s])
    assert np.array_equal(s_b[w["slot_idx"][3]], st_f[w["slot_idx"][3]])


def pin_bf16_work():
    """Verify page, work_dtype bfloat16: bf16 per-token inputs widen exactly
    and the output is rounded once, so the result is torch's bf16 cast of the
    float32 run on the widened inputs, and the state is that run's, bit for
    bit (forward, verify and fused entries)."""
    w = small_packed(29, [3, 0, 6, 2], K=8, V=8, state_dtype="bf16")
    wb = wl.bf16_work(w)
    ww = dict(wb, **{k: wl.bf16_bits_to_f32(wb[k]) for k in ("qkv", "decay", "beta")})
    out_b, st_b = run_fwd(wb)
    out_w, st_w = run_fwd(ww)
    assert out_b.dtype == np.uint16
    assert np.array_equal(out_b, wl.to_bf16_bits(out_w))
    assert np.array_equal(st_b, st_w)
    rng = _rng(30)
    g = wl.gdp_inputs(rng, B=3, S_draft=2, M=2, H=2, HV=4, K=8, V=8, slots=4, pad_frac=0.3,
                      state_sigma=0.2)
    gb = wl.bf16_work(g)
    gw = dict(gb, **{k: wl.bf16_bits_to_f32(gb[k]) for k in ("q", "k", "v", "g", "beta")})
    keys = ("q", "k", "v", "g", "beta", "state", "state_indices", "intermediate_states",
            "steps_per_token", "use_qk_l2norm_in_kernel", "scale")
    o_b, s_b, i_b = oracle.fused_recurrent_update(**{k: gb[k] for k in keys})
    o_w, s_w, i_w = oracle.fused_recurrent_update(**{k: gw[k] for k in keys})
    assert np.array_equal(o_b, wl.to_bf16_bits(o_w))
    assert np.array_equal(s_b, s_w) and np.array_equal(i_b, i_w)


def _conv_inputs(seed, lengths, C=6, W=4, slots=5):
    rng = _rng(seed)
    T = int(sum(lengths))
    off = np.zeros(len(lengths) + 1, np.uint32)
    off[1:] = np.cumsum(lengths)
    x = rng.standard_normal((T, C)).astype(np.float32)
    w = rng.standard_normal((C, W)).astype(np.float32)
    b = rng.standard_normal(C).astype(np.float32)
    st = rng.standard_normal((slots, W - 1, C)).astype(np.float32)
    sl = rng.choice(slots, size=len(lengths), replace=False).astype(np.uint32)
    return dict(x=x, weight=w, bias=b, conv_state=st, slot_idx=sl, row_offsets=off)


def pin_conv_taps():
    """Causal Conv1d reading: a one-hot filter at tap j delays the input by
    W-1-j tokens, the first ones coming from the slot's history; the new
    history is the last W-1 inputs of history ++ row."""
    lengths = [5, 1, 0, 2]
    W, C = 4, 6
    a = _conv_inputs(31, lengths, C=C, W=W)
    off = a["row_offsets"]
    for j in range(W):
        w = np.zeros((C, W), np.float32)
        w[:, j] = 1.0
        out, st = oracle.causal_conv1d(**dict(a, weight=w, bias=None))
        d = W - 1 - j
        for b, L in enumerate(lengths):
            hist = a["conv_state"][a["slot_idx"][b]]
            seq = np.concatenate([hist, a["x"][off[b]:off[b + 1]]])
            for t in range(L):
                assert np.array_equal(out[off[b] + t], seq[W - 1 + t - d]), (j, b, t)
            want = seq[-(W - 1):] if L else hist
            assert np.array_equal(st[a["slot_idx"][b]], want), (j, b)


def pin_conv_numpy():
    """With zero history the output is the per-channel full convolution of the
    row with the reversed filter, plus bias (numpy's convolve, float64)."""
    lengths = [7, 3, 12]
    a = _conv_inputs(32, lengths, W=3)
    out, _ = oracle.causal_conv1d(**dict(a, conv_state=None))
    off = a["row_offsets"]
    for b, L in enumerate(lengths):
        for c in range(a["x"].shape[1]):
            xr = a["x"][off[b]:off[b + 1], c].astype(np.float64)
            want = np.convolve(xr, a["weight"][c, ::-1].astype(np.float64))[:L] + a["bias"][c]
            _close(out[off[b]:off[b + 1], c], want, 1e-6, f"conv row {b} ch {c}")


def pin_conv_continuity():
    """Splitting every row in two calls (the first updating the history)
    gives the outputs and history of one call over the whole rows, bit for
    bit; padding rows give +0.0 and touch nothing; SiLU is y * sigmoid(y)."""
    lengths = [9, 4, 6]
    a = _conv_inputs(33, lengths, W=4)
    off = a["row_offsets"].astype(np.int64)
    whole, st_whole = oracle.causal_conv1d(**a)
    cut = [3, 1, 6]
    for part in (0, 1):
        rows = [np.arange(off[b], off[b] + cut[b]) if part == 0 else
                np.arange(off[b] + cut[b], off[b + 1]) for b in range(3)]
        o2 = np.zeros(len(lengths) + 1, np.uint32)
        o2[1:] = np.cumsum([len(r) for r in rows])
        sub = dict(a, x=a["x"][np.concatenate(rows)], row_offsets=o2,
                   conv_state=a["conv_state"] if part == 0 else st_part)
        out_p, st_part = oracle.causal_conv1d(**sub)
        assert np.array_equal(out_p, whole[np.concatenate(rows)]), part
    assert np.array_equal(st_part, st_whole)
    pad = dict(a, slot_idx=a["slot_idx"].copy())
    pad["slot_idx"][1] = 0xFFFFFFFF
    out_pad, st_pad = oracle.causal_conv1d(**pad)
    z = out_pad[off[1]:off[2]]
    assert np.array_equal(z, np.zeros_like(z)) and not np.signbit(z).any()
    assert np.array_equal(st_pad[a["slot_idx"][1]], a["conv_state"][a["slot_idx"][1]])
    y, _ = oracle.causal_conv1d(**a)
    s_, _ = oracle.causal_conv1d(**a, silu=True)
    y64 = y.astype(np.float64)
    _close(s_, y64 / (1.0 + np.exp(-y64)), 1e-6, "silu")
    xb = wl.to_bf16_bits(a["x"])
    sb = wl.to_bf16_bits(a["conv_state"])
    ob, stb = oracle.causal_conv1d(**dict(a, x=xb, conv_state=sb))
    ow, stw = oracle.causal_conv1d(**dict(a, x=wl.bf16_bits_to_f32(xb),
                                          conv_state=wl.bf16_bits_to_f32(sb)))
    assert np.array_equal(ob, wl.to_bf16_bits(ow))
    assert np.array_equal(stb, wl.to_bf16_bits(stw))


def pin_golden_hand():
    """tests/golden/hand_k2_v2.json: a two-token example worked by hand in exact
    dyadic arithmetic."""
    with open(os.path.join(HERE, "golden", "hand_k2_v2.json")) as f:
        g = json.load(f)
    toks = g["tokens"]
    qkv = np.array([t["q"] + t["k"] + t["v"] for t in toks], np.float32)
    decay = np.array([[t["decay"]] for t in toks], np.float32)
    beta = np.array([[t["beta"]] for t in toks], np.float32)
    state = np.array(g["initial_state"], np.float32).reshape(1, 1, 2, 2)
    out, st = oracle.recurrence_fwd(
        qkv=qkv, decay=decay, beta=beta, state=state, slot_idx=np.array([0], np.uint32),
        row_offsets=np.array([0, 2], np.uint32), num_value_heads=1, num_key_heads=1,
        scale=g["layout"]["scale"], l2norm=False)
    assert np.array_equal(out, np.array(g["expected_out"], np.float32)), out
    assert np.array_equal(st[0, 0], np.array(g["expected_state"], np.float32)), st


def pin_bf16_rounding():
    """The oracle's bf16 store rounds like torch's float32 -> bfloat16 cast
    (nearest even), including exact ties."""
    rng = _rng(25)
    x = np.concatenate([
        rng.standard_normal(4096).astype(np.float32),
        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0, -0.0, 1e-30,
                  3.0e38, np.inf, -np.inf], np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_round(x)
    assert np.array_equal(got, want)
    nan = oracle.bf16_round(np.array([np.nan], np.float32))
    assert wl.bf16_bits_to_f32(nan)[0] != wl.bf16_bits_to_f32(nan)[0]


ALL_PINS = [pin_dense_fp64, pin_dense_unrolled, pin_beta_zero_decay_only, pin_delta_retrieval,
            pin_scalar_state, pin_gather_probe, pin_scatter_probe, pin_linearity_pow2,
            pin_verify_fold_identities, pin_replicated_heads, pin_fused_matches_packed,
            pin_snapshots, pin_snapshot_rollback, pin_per_v_beta, pin_bf16_ring, pin_bf16_work,
            pin_conv_taps, pin_conv_numpy, pin_conv_continuity, pin_golden_hand,
            pin_bf16_rounding]
