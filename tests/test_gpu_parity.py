"""GPU parity: the HIP library, called through its C ABI, against the CPU
oracle on the same seeded inputs, plus the bit-exact identities the pages
state, checked on the GPU path itself."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import gated_delta_rule_loop_amd as gdr
import oracle
from gated_delta_rule_loop_amd import workloads as wl
from tests import gpu_harness as H
from tests import oracle_pins as P

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-parity]", *a, flush=True)
    sys.stdout.flush()


def oracle_fwd(w, state=None, **kw):
    args = {k: w[k] for k in ("qkv", "decay", "beta", "slot_idx", "row_offsets",
                              "num_value_heads", "num_key_heads")}
    args["state"] = w["state"] if state is None else state
    if "scale" in w:
        args["scale"] = w["scale"]
    args.update(kw)
    return oracle.recurrence_fwd(**args)


def touched(w):
    s = np.asarray(w["slot_idx"]).astype(np.int64)
    return s[s != wl.PAD_SLOT_U32]


def check_fwd_against_oracle(w, name, gpu=None, **kw):
    out_g, st_g = H.gpu_fwd(w, **kw) if gpu is None else gpu
    out_r, st_r = oracle_fwd(w, **{k: v for k, v in kw.items() if k != "out"})
    err = H.assert_close(out_g, out_r, f"{name} output")
    bf16 = w["state"].dtype == np.uint16
    unr = None
    if bf16:
        _, unr = oracle_fwd(w, state=H.f32_pool(w["state"]),
                            **{k: v for k, v in kw.items() if k != "out"})
    sl = touched(w)
    ties = H.assert_state_close(st_g[sl], st_r[sl], f"{name} state",
                                None if unr is None else unr[sl])
    others = np.setdiff1d(np.arange(w["state"].shape[0]), sl)
    assert np.array_equal(st_g[others], w["state"][others]), f"{name}: untouched slots changed"
    say(f"{name}: out rel err {err:.2e}, state ties {ties}")
    return out_g, st_g


# ------------------------------------------------------------ the configs ---

def test_tiny_ragged_fwd():
    say("tiny ragged forward: B=2 L=[3,5] nk=1 nv=2 K=V=16 f32 pool")
    w = wl.tiny_ragged()
    check_fwd_against_oracle(w, "tiny")


def test_decode_step():
    say("decode step: B=256 x 1 token nk=16 nv=32 K=V=128 bf16 pool 512")
    w = wl.decode_step()
    check_fwd_against_oracle(w, "decode")


def sub_packed(w, rows, key_heads):
    """The packed workload restricted to some rows and key heads (slicing only)."""
    nk, nv = w["num_key_heads"], w["num_value_heads"]
    G = nv // nk
    K, V = w["state"].shape[2], w["state"].shape[3]
    vheads = [h * G + m for h in key_heads for m in range(G)]
    off = w["row_offsets"].astype(np.int64)
    toks = np.concatenate([np.arange(off[b], off[b + 1]) for b in rows])
    cols = ([np.arange(h * K, (h + 1) * K) for h in key_heads] +
            [nk * K + np.arange(h * K, (h + 1) * K) for h in key_heads] +
            [2 * nk * K + np.arange(hv * V, (hv + 1) * V) for hv in vheads])
    cols = np.concatenate(cols)
    lens = [off[b + 1] - off[b] for b in rows]
    new_off = np.zeros(len(rows) + 1, np.uint32)
    new_off[1:] = np.cumsum(lens)
    sub = dict(qkv=np.ascontiguousarray(w["qkv"][np.ix_(toks, cols)]),
               decay=np.ascontiguousarray(w["decay"][np.ix_(toks, vheads)]),
               beta=np.ascontiguousarray(w["beta"][np.ix_(toks, vheads)]),
               state=np.ascontiguousarray(w["state"][:, vheads]),
               slot_idx=w["slot_idx"][rows].copy(), row_offsets=new_off,
               num_key_heads=len(key_heads), num_value_heads=len(vheads))
    return sub, toks, vheads


def test_ragged_prefill_full():
    """Config 2 in full: every output of every row and value head, and every
    touched state, against the oracle (its (row, value head) items run on a
    few host threads; the results do not depend on the thread count)."""
    w = wl.ragged_prefill()
    lens = np.diff(w["row_offsets"].astype(np.int64))
    threads = oracle.default_threads()
    say(f"ragged prefill: B=8 lengths {lens.tolist()}, all {int(lens.sum())} tokens x 32 "
        f"value heads against the oracle ({threads} host threads)")
    out_g, st_g = H.gpu_fwd(w)
    out_r, st_r = oracle_fwd(w, threads=threads)
    err = H.assert_close(out_g, out_r, "prefill output")
    _, unr = oracle_fwd(w, state=H.f32_pool(w["state"]), threads=threads)
    sl = touched(w)
    ties = H.assert_state_close(st_g[sl], st_r[sl], "prefill state", unr[sl])
    others = np.setdiff1d(np.arange(64), sl)
    assert np.array_equal(st_g[others], w["state"][others]), "prefill: untouched slots changed"
    # the same call on a float32 copy of the pool: identical outputs, and the
    # bf16 states are the float32 states rounded to nearest even
    out_32, st_32 = H.gpu_fwd(dict(w, state=H.f32_pool(w["state"])))
    assert np.array_equal(out_32.view(np.uint32), out_g.view(np.uint32))
    assert np.array_equal(wl.to_bf16_bits(st_32[sl]), st_g[sl])
    gap = H.record_fp32_gap("prefill", st_32[sl], unr[sl])
    say(f"prefill: out rel err {err:.2e}, state ties {ties}, float32 state gap {gap:.1e}")


def test_float32_disagreement_decode_verify_gdp():
    """The float32 gap between the GPU and the oracle (different reduction
    order) on the decode step, the verify window's committed rows and the GDP
    decode, measured with float32 pools; it bounds how close to a bf16
    rounding midpoint an accepted tie must lie."""
    w = wl.decode_step()
    sl = touched(w)
    w32 = dict(w, state=H.f32_pool(w["state"]))
    _, st_g = H.gpu_fwd(w32)
    _, st_r = oracle_fwd(w32, threads=oracle.default_threads())
    g1 = H.record_fp32_gap("decode", st_g[sl], st_r[sl])
    v = wl.verify_window()
    v32 = dict(v, state=H.f32_pool(v["state"]))
    _, st_g, _ = H.gpu_verify(v32)
    _, st_r, _ = verify_oracle(v32)
    lens = np.diff(v["row_offsets"].astype(np.int64))
    long_slots = v["slot_idx"][lens > v["ring"].shape[2]].astype(np.int64)
    g2 = H.record_fp32_gap("verify commit", st_g[long_slots], st_r[long_slots])
    f = wl.gdp_decode()
    f32 = dict(f, state=H.f32_pool(f["state"]),
               intermediate_states=np.zeros(f["intermediate_states"].shape, np.float32))
    _, st_g, in_g = H.gpu_fused(f32)
    _, st_u, in_u = fused_oracle(f, f32=True)
    act = f["state_indices"][f["state_indices"] >= 0].astype(np.int64)
    g3 = H.record_fp32_gap("gdp state", st_g[act], st_u[act])
    g4 = H.record_fp32_gap("gdp snapshots", in_g[act], in_u[act])
    say(f"float32 state gap: decode {g1:.1e}, verify commit {g2:.1e}, gdp {g3:.1e} / {g4:.1e}")


def verify_oracle(w, state=None):
    args = {k: w[k] for k in ("qkv", "decay", "beta", "slot_idx", "row_offsets",
                              "num_value_heads", "num_key_heads", "ring", "ring_slot_idx")}
    args["state"] = w["state"] if state is None else state
    return oracle.recurrence_verify_ring(**args)


def test_verify_window_and_fold():
    w = wl.verify_window()
    lens = np.diff(w["row_offsets"].astype(np.int64))
    ring_len = w["ring"].shape[2]
    say(f"verify window + fold: B=64 windows in [1,12] ring_len {ring_len}, "
        f"{int((lens > ring_len).sum())} long rows")
    out_g, st_g, ring_g = H.gpu_verify(w)
    out_r, st_r, ring_r = verify_oracle(w)
    H.assert_close(out_g, out_r, "verify verify output")
    # GPU identity: verify output == forward output, bit for bit
    out_f, st_f = H.gpu_fwd(w)
    assert np.array_equal(out_g.view(np.uint32), out_f.view(np.uint32)), "verify != fwd output"
    _, unr_v, _ = verify_oracle(w, state=H.f32_pool(w["state"]))
    for b, L in enumerate(lens):
        s = w["slot_idx"][b]
        if L <= ring_len:   # state untouched, bit for bit
            assert np.array_equal(st_g[s], w["state"][s]), f"row {b}: verify wrote the state"
        else:               # committed like the forward, bit for bit, and no records
            assert np.array_equal(st_g[s], st_f[s]), f"row {b}: long row commit != fwd"
            H.assert_state_close(st_g[s], st_r[s], f"verify row {b} commit", unr_v[s])
            assert not ring_g[w["ring_slot_idx"][b]].any(), f"row {b}: long row recorded"
    # ring records against the oracle's (only entries the rows wrote)
    G = 2
    K = V = 128
    for b, L in enumerate(lens):
        if L > ring_len:
            continue
        rr = w["ring_slot_idx"][b]
        got = ring_g[rr, :, :L, :K + G * (V + 1)]
        ref = ring_r[rr, :, :L, :K + G * (V + 1)]
        H.assert_close(got, ref, f"verify ring row {b}")
    # fold with the configured accepted counts
    acc = w["accepted"]
    st_fold_g = H.gpu_fold(w, st_g, ring_g, acc)
    st_fold_r = oracle.state_fold(state=st_r, slot_idx=w["slot_idx"], ring=ring_r,
                                  ring_slot_idx=w["ring_slot_idx"], accepted=acc,
                                  num_value_heads=32, num_key_heads=16)
    unr_f = oracle.state_fold(state=unr_v, slot_idx=w["slot_idx"], ring=ring_r,
                              ring_slot_idx=w["ring_slot_idx"], accepted=acc,
                              num_value_heads=32, num_key_heads=16)
    sl = touched(w)
    ties = H.assert_state_close(st_fold_g[sl], st_fold_r[sl], "verify fold state", unr_f[sl])
    # GPU identity: fold(n) == forward over the first n tokens, bit for bit
    pre_len = [int(a) for a in acc]
    off = w["row_offsets"].astype(np.int64)
    keep = np.concatenate([np.arange(off[b], off[b] + pre_len[b]) for b in range(64)])
    offs = np.zeros(65, np.uint32)
    offs[1:] = np.cumsum(pre_len)
    pre = dict(w, qkv=w["qkv"][keep], decay=w["decay"][keep], beta=w["beta"][keep],
               row_offsets=offs)
    _, st_pre = H.gpu_fwd(pre)
    for b, L in enumerate(lens):
        s = w["slot_idx"][b]
        assert np.array_equal(st_fold_g[s], st_pre[s]), f"row {b}: fold({acc[b]}) != fwd prefix"
    say(f"verify: verify/fold parity ok, fold ties {ties}")


def fused_oracle(w, f32=False):
    args = {k: w[k] for k in ("q", "k", "v", "g", "beta", "state", "state_indices",
                              "intermediate_states", "steps_per_token",
                              "use_qk_l2norm_in_kernel", "scale")}
    if f32:
        args["state"] = H.f32_pool(w["state"])
        inter = w["intermediate_states"]
        args["intermediate_states"] = np.zeros(inter.shape, np.float32)
    return oracle.fused_recurrent_update(**args)


def test_gdp_decode():
    w = wl.gdp_decode()
    idx = w["state_indices"]
    say(f"GDP decode: B=128 T=8 spt=2, {int((idx < 0).sum())} padding rows")
    o_g, st_g, inter_g = H.gpu_fused(w)
    o_r, st_r, inter_r = fused_oracle(w)
    o_u, st_u, inter_u = fused_oracle(w, f32=True)
    err = H.assert_close(o_g, o_r, "gdp output")
    pad = idx < 0
    assert np.array_equal(o_g[pad].view(np.uint32), np.zeros_like(o_g[pad]).view(np.uint32))
    sl = idx[~pad].astype(np.int64)
    ties = H.assert_state_close(st_g[sl], st_r[sl], "gdp state", st_u[sl])
    ties += H.assert_state_close(inter_g[sl], inter_r[sl], "gdp snapshots", inter_u[sl])
    others = np.setdiff1d(np.arange(256), sl)
    assert np.array_equal(st_g[others], w["state"][others])
    assert np.array_equal(inter_g[others], w["intermediate_states"][others])
    # GPU identity: last snapshot == final state, bit for bit
    assert np.array_equal(inter_g[sl, -1], st_g[sl])
    # GDP caller slicing: the answer of draft token i is on copy M-1
    M = w["steps_per_token"]
    assert o_g[:, M - 1::M].shape[1] == 4
    say(f"gdp: out rel err {err:.2e}, state+snapshot ties {ties}")


def test_snapshot_equals_prefix_run():
    """intermediate[slot, i] equals the state of a GPU run over the first
    (i+1)*spt steps, bit for bit."""
    rng = np.random.Generator(np.random.PCG64(77))
    w = wl.gdp_inputs(rng, B=9, S_draft=3, M=2, H=4, HV=8, K=128, V=128, slots=12,
                      pad_frac=0.2, state_sigma=0.05)
    say("snapshot == prefix run, B=9 T=6 spt=2")
    _, st_full, inter = H.gpu_fused(w)
    M = w["steps_per_token"]
    for i in range(3):
        n = (i + 1) * M
        sub = dict(w, q=w["q"][:, :n], k=w["k"][:, :n], v=w["v"][:, :n], g=w["g"][:, :n],
                   beta=w["beta"][:, :n], intermediate_states=None)
        _, st_i, _ = H.gpu_fused(sub)
        for idx in w["state_indices"]:
            if idx >= 0:
                assert np.array_equal(inter[idx, i], st_i[idx]), (i, idx)


# --------------------------------------------------- exact probes on GPU ---

def test_gather_probe_gpu():
    rng = np.random.Generator(np.random.PCG64(17))
    nk, nv, K, V = 2, 6, 16, 16
    w = P.small_packed(17, [3, 0, 5, 2], nk=nk, nv=nv, K=K, V=V, slots=9, state_dtype="bf16")
    T = w["qkv"].shape[0]
    w["decay"][:] = 1.0
    w["beta"][:] = 0.0
    istar = rng.integers(0, K, size=(T, nk))
    w["qkv"][:, :nk * K] = 0.0
    for t in range(T):
        for h in range(nk):
            w["qkv"][t, h * K + istar[t, h]] = 1.0
    out, st = H.gpu_fwd(w, scale=1.0, l2norm=False)
    S0 = H.as_f32(w["state"])
    G = nv // nk
    for b in range(4):
        for t in range(w["row_offsets"][b], w["row_offsets"][b + 1]):
            for hv in range(nv):
                want = S0[w["slot_idx"][b], hv, istar[t, hv // G], :]
                assert np.array_equal(out[t, hv * V:(hv + 1) * V], want), (b, t, hv)
    assert np.array_equal(st, w["state"])


def test_scatter_probe_gpu():
    rng = np.random.Generator(np.random.PCG64(18))
    nk, nv, K, V = 4, 8, 128, 128
    w = P.small_packed(18, [2, 4, 1], nk=nk, nv=nv, K=K, V=V, slots=8, state_dtype="bf16")
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
    _, st = H.gpu_fwd(w, scale=1.0, l2norm=False)
    S1 = H.as_f32(st)
    G = nv // nk
    for b in range(3):
        tl = int(w["row_offsets"][b + 1]) - 1
        for hv in range(nv):
            want = np.zeros((K, V), np.float32)
            want[istar[tl, hv // G]] = w["qkv"][tl, 2 * nk * K + hv * V:2 * nk * K + (hv + 1) * V]
            assert np.array_equal(S1[w["slot_idx"][b], hv], want), (b, hv)
    others = np.setdiff1d(np.arange(8), w["slot_idx"])
    assert np.array_equal(st[others], w["state"][others])


def test_linearity_pow2_gpu():
    w = P.small_packed(19, [3, 6, 1, 40], nk=2, nv=4, K=128, V=128, slots=6, state_dtype="bf16")
    out1, st1 = H.gpu_fwd(w)
    w2 = dict(w, qkv=w["qkv"].copy(), state=wl.to_bf16_bits(2.0 * H.as_f32(w["state"])))
    w2["qkv"][:, 2 * 2 * 128:] *= 2.0
    out2, st2 = H.gpu_fwd(w2)
    assert np.array_equal(out2, 2.0 * out1)
    assert np.array_equal(H.as_f32(st2), 2.0 * H.as_f32(st1))


def test_replicated_heads_gpu():
    nk, nv, K, V = 2, 4, 128, 128
    w = P.small_packed(22, [3, 5, 20], nk=nk, nv=nv, K=K, V=V, slots=4, state_dtype="bf16")
    out1, st1 = H.gpu_fwd(w)
    x = w["qkv"]
    q = x[:, :nk * K].reshape(-1, nk, K)
    k = x[:, nk * K:2 * nk * K].reshape(-1, nk, K)
    rep = np.arange(nv) // (nv // nk)
    x2 = np.concatenate([q[:, rep].reshape(len(x), -1), k[:, rep].reshape(len(x), -1),
                         x[:, 2 * nk * K:]], axis=1)
    out2, st2 = H.gpu_fwd(dict(w, qkv=np.ascontiguousarray(x2), num_key_heads=nv))
    assert np.array_equal(out1.view(np.uint32), out2.view(np.uint32))
    assert np.array_equal(st1, st2)


def test_launch_shape_independence():
    """A row gives the same bits whether the batch around it makes the host
    pick the wide (few tokens per row) or the narrow (long rows) tiling."""
    w = P.small_packed(31, [1, 1, 1, 37], nk=2, nv=4, K=128, V=128, slots=6, state_dtype="bf16")
    out_a, st_a = H.gpu_fwd(w)   # 40 tokens / 4 rows -> wide tiles
    sub, toks, _ = sub_packed(w, [3], [0, 1])
    out_b, st_b = H.gpu_fwd(sub)  # 37 tokens / 1 row -> narrow tiles
    assert np.array_equal(out_a[toks].view(np.uint32), out_b.view(np.uint32))
    s = w["slot_idx"][3]
    assert np.array_equal(st_a[s], st_b[s])


@pytest.mark.parametrize("K,ring_len", [(128, 6), (256, 6), (128, 19), (256, 19), (64, 19), (16, 19)])
def test_fold_equals_forward_prefix_every_n(K, ring_len):
    """fold(n) equals the forward pass over the first n tokens, bit for bit,
    for every n; a ring longer than 8 tokens folds in several LDS stages."""
    lengths = [1, 6, 3, 9, 5] if ring_len < 9 else [1, 19, 8, 20, 17]
    nk, nv, V = 2, 4, K
    w = P.small_packed(40, lengths, nk=nk, nv=nv, K=K, V=V, slots=7, state_dtype="bf16")
    stride = wl.ring_record_stride(nv // nk, K, V)
    w["ring"] = np.zeros((5, nk, ring_len, stride), np.float32)
    w["ring_slot_idx"] = np.array([4, 0, 2, 1, 3], np.uint32)
    _, st_v, ring_v = H.gpu_verify(w)
    off = w["row_offsets"].astype(np.int64)
    for n in range(0, max(lengths) + 1):
        acc = np.array([min(n, L) if L <= ring_len else L for L in lengths], np.uint32)
        folded = H.gpu_fold(w, st_v, ring_v, acc)
        keep = np.concatenate([np.arange(off[b], off[b] + acc[b]) for b in range(5)])
        offs = np.zeros(6, np.uint32)
        offs[1:] = np.cumsum(acc)
        _, st_pre = H.gpu_fwd(dict(w, qkv=w["qkv"][keep], decay=w["decay"][keep],
                                   beta=w["beta"][keep], row_offsets=offs))
        for b in range(5):
            s = w["slot_idx"][b]
            assert np.array_equal(folded[s], st_pre[s]), (n, b)


# ------------------------------------------------------------ edge cases ---

@pytest.mark.parametrize("K", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("state_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("lengths", [[0, 3, 1, 7], [25, 0, 19], [40, 0, 33]])
def test_small_shapes(K, state_dtype, lengths):
    say(f"small shapes K={K} {state_dtype} lengths {lengths}")
    w = P.small_packed(50 + K, lengths, nk=2, nv=4, K=K, V=K, slots=5, state_dtype=state_dtype,
                       sigma=0.1)
    check_fwd_against_oracle(w, f"K{K}-{state_dtype}-{lengths}")


def test_padding_rows_packed_entries():
    w = P.small_packed(60, [2, 3, 4], nk=2, nv=4, K=128, V=128, slots=5, state_dtype="bf16")
    w["slot_idx"][1] = wl.PAD_SLOT_U32
    out_g, st_g = H.gpu_fwd(w)
    t0, t1 = w["row_offsets"][1], w["row_offsets"][2]
    assert np.array_equal(out_g[t0:t1].view(np.uint32), np.zeros((t1 - t0, 512), np.uint32))
    check_fwd_against_oracle(w, "padding")


def test_strided_views():
    """Non-contiguous inputs: qkv rows inside a wider buffer, gates as column
    views, the state pool as a head slice of a larger pool."""
    import torch
    import gated_delta_rule_loop_amd as gdr
    w = P.small_packed(61, [4, 1, 6], nk=2, nv=4, K=64, V=64, slots=5, state_dtype="bf16")
    T = w["qkv"].shape[0]
    wide = np.zeros((T, w["qkv"].shape[1] + 64), np.float32)
    wide[:, 32:32 + w["qkv"].shape[1]] = w["qkv"]
    gates = np.zeros((T, 8), np.float32)
    gates[:, 0:4] = w["decay"]
    gates[:, 4:8] = w["beta"]
    big = np.zeros((5, 6, 64, 64), np.uint16)
    big[:, 1:5] = w["state"]
    qkv_t = H.dev(wide)[:, 32:32 + w["qkv"].shape[1]]
    g_t = H.dev(gates)
    st_t = H.dev(big)
    out = torch.full((T, 256), float("nan"), device="cuda")
    gdr.gdr_recurrence_fwd(out, st_t[:, 1:5], H.dev(w["slot_idx"]), qkv_t, g_t[:, 0:4],
                           g_t[:, 4:8], H.dev(w["row_offsets"]), num_value_heads=4,
                           num_key_heads=2)
    torch.cuda.synchronize()
    big_after = H.host(st_t)
    check_fwd_against_oracle(w, "strided", gpu=(H.host(out), big_after[:, 1:5]))
    assert np.array_equal(big_after[:, 0], big[:, 0]) and np.array_equal(big_after[:, 5], big[:, 5])


def test_fused_dense_and_varlen_paths():
    """Fused update without a cache (initial/final state, zeros) and with
    cu_seqlens, against the oracle."""
    rng = np.random.Generator(np.random.PCG64(62))
    w = wl.gdp_inputs(rng, B=3, S_draft=5, M=1, H=2, HV=4, K=64, V=64, slots=4, pad_frac=0.0,
                      state_sigma=0.1, state_dtype="f32")
    init = w["state"][:3].copy()
    base = dict(q=w["q"], k=w["k"], v=w["v"], g=w["g"], beta=w["beta"], scale=None,
                use_qk_l2norm_in_kernel=True)
    for kind in ("zeros", "initial"):
        extra = dict(output_final_state=True)
        if kind == "initial":
            extra["initial_state"] = init
        o_g, fin_g, _ = H.gpu_fused(base, **extra)
        o_r, fin_r, _ = oracle.fused_recurrent_update(**base, **extra)
        H.assert_close(o_g, o_r, f"fused {kind} output")
        H.assert_close(fin_g, fin_r, f"fused {kind} final state")
    # varlen: B=1 with cu_seqlens over the flattened tokens, pool + indices
    T = 15
    cu = np.array([0, 4, 4, 11, 15], np.int32)
    vl = dict(q=w["q"].reshape(1, T, 2, 64), k=w["k"].reshape(1, T, 2, 64),
              v=w["v"].reshape(1, T, 4, 64), g=w["g"].reshape(1, T, 4),
              beta=w["beta"].reshape(1, T, 4), use_qk_l2norm_in_kernel=True, cu_seqlens=cu,
              state=w["state"], state_indices=np.array([2, 0, -1, 3], np.int32))
    o_g, st_g, _ = H.gpu_fused(vl)
    o_r, st_r, _ = oracle.fused_recurrent_update(**vl)
    H.assert_close(o_g, o_r, "varlen output")
    H.assert_close(st_g, st_r, "varlen state")
    assert not o_g[0, 4:11].any()


def test_snapshot_rollback_gpu():
    """Rollback after n accepted drafts == a GPU run over the first n * spt
    steps (bit for bit), and == the oracle's copy on the same arrays; n = 0,
    n past the buffer and padding leave the state alone."""
    import torch
    import gated_delta_rule_loop_amd as gdr
    rng = np.random.Generator(np.random.PCG64(78))
    w = wl.gdp_inputs(rng, B=10, S_draft=3, M=2, H=4, HV=8, K=128, V=128, slots=14,
                      pad_frac=0.2, state_sigma=0.05)
    say("snapshot rollback, B=10 T=6 spt=2")
    _, st, inter = H.gpu_fused(w)
    idx = w["state_indices"]
    acc = np.full(len(idx), 2, np.int32)
    active = np.flatnonzero(idx >= 0)
    acc[active] = np.resize(np.array([1, 2, 3, 0, 4], np.int32), len(active))
    st_t = H.dev(st)
    gdr.gdr_snapshot_rollback(st_t, H.dev(idx.astype(np.int32)), H.dev(inter), H.dev(acc))
    torch.cuda.synchronize()
    rolled = H.host(st_t)
    want = oracle.snapshot_rollback(state=st, state_indices=idx, intermediate_states=inter,
                                    accepted=acc)
    assert np.array_equal(rolled, want)
    M = w["steps_per_token"]
    for b, i in enumerate(idx):
        n = int(acc[b])
        if i < 0 or not 1 <= n <= 3:
            if i >= 0:
                assert np.array_equal(rolled[i], st[i])
            continue
        sub = dict(w, q=w["q"][:, :n * M], k=w["k"][:, :n * M], v=w["v"][:, :n * M],
                   g=w["g"][:, :n * M], beta=w["beta"][:, :n * M], intermediate_states=None)
        _, st_n, _ = H.gpu_fused(sub)
        assert np.array_equal(rolled[i], st_n[i]), (b, n)


# ------------------------------------------- per-column beta, bf16 ring ---

@pytest.mark.parametrize("case", [
    # (B, S_draft, M, H, HV, K, state dtype, snapshots): fused short rows,
    # decode (one step), long rows, and the smaller head dims
    (16, 4, 2, 4, 8, 128, "bf16", True),
    (24, 1, 1, 4, 8, 128, "bf16", False),
    (3, 20, 2, 2, 4, 128, "f32", True),
    (5, 3, 2, 2, 4, 64, "f32", True),
    (4, 6, 1, 2, 8, 32, "bf16", False),
    (6, 2, 3, 1, 2, 16, "f32", True),
], ids=lambda c: "B{}_S{}_M{}_H{}_HV{}_K{}_{}_{}".format(*c[:7], "snap" if c[7] else "nosnap"))
def test_per_column_beta_gpu(case):
    """Fused update with beta [B, T, HV, V] against the oracle; a per-column
    beta whose columns are equal gives the head-wise result bit for bit."""
    B, S, M, Hh, HV, K, sd, snap = case
    rng = np.random.Generator(np.random.PCG64(90 + K + B))
    w = wl.gdp_inputs(rng, B=B, S_draft=S, M=M, H=Hh, HV=HV, K=K, V=K, slots=B + 3,
                      pad_frac=0.15, state_sigma=0.1, state_dtype=sd, beta_per_v=True)
    if not snap:
        w["intermediate_states"] = None
    say(f"per-column beta: {case}")
    o_g, st_g, inter_g = H.gpu_fused(w)
    o_r, st_r, inter_r = fused_oracle(w)
    st_u = inter_u = None  # unrounded oracle states, to judge bf16 rounding ties
    if sd == "bf16" and snap:
        _, st_u, inter_u = fused_oracle(w, f32=True)
    elif sd == "bf16":
        _, st_u, _ = oracle.fused_recurrent_update(**{**{k: w[k] for k in (
            "q", "k", "v", "g", "beta", "state_indices", "steps_per_token",
            "use_qk_l2norm_in_kernel", "scale")}, "state": H.f32_pool(w["state"])})
    err = H.assert_close(o_g, o_r, "per-column beta output")
    idx = w["state_indices"]
    sl = idx[idx >= 0].astype(np.int64)
    H.assert_state_close(st_g[sl], st_r[sl], "per-column beta state",
                         None if st_u is None else st_u[sl])
    if snap:
        H.assert_state_close(inter_g[sl], inter_r[sl], "per-column beta snapshots",
                             None if inter_u is None else inter_u[sl])
    head = np.ascontiguousarray(w["beta"][..., 0])
    flat = np.ascontiguousarray(np.repeat(head[..., None], K, axis=-1))
    o1, st1, i1 = H.gpu_fused(w, beta=head)
    o2, st2, i2 = H.gpu_fused(w, beta=flat)
    bits = lambda a: a.view(np.uint32 if a.dtype == np.float32 else np.uint16)  # noqa: E731
    assert np.array_equal(bits(o1), bits(o2))
    assert np.array_equal(bits(st1), bits(st2))
    if snap:  # untouched entries hold NaN sentinels: compare bits
        assert np.array_equal(bits(i1), bits(i2))
    say(f"per-column beta: out rel err {err:.2e}")


def test_bf16_ring_verify_and_fold():
    """Verify with a bf16 ring: output and state as with a float32 ring, bit
    for bit; every record is the float32 record rounded to nearest even; the
    fold of the bf16 ring equals the fold of its widened values bit for bit
    and the oracle's bf16-ring fold within tolerance."""
    import torch
    w = wl.verify_window()
    lens = np.diff(w["row_offsets"].astype(np.int64))
    ring_len = w["ring"].shape[2]
    ring_b0 = np.zeros(w["ring"].shape, np.uint16)
    say("bf16 ring: verify window B=64, ring_len 8")
    out_f, st_f, ring_f = H.gpu_verify(w)
    out_b, st_b, ring_b = H.gpu_verify(w, ring=ring_b0)
    assert np.array_equal(out_b.view(np.uint32), out_f.view(np.uint32))
    assert np.array_equal(st_b, st_f)
    want = torch.from_numpy(ring_f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ring_b, want), "bf16 ring != rounded float32 ring"
    acc = w["accepted"]
    fold_b = H.gpu_fold(w, st_b, ring_b, acc)
    fold_w = H.gpu_fold(w, st_b, np.ascontiguousarray(wl.bf16_bits_to_f32(ring_b)), acc)
    assert np.array_equal(fold_b, fold_w), "bf16-ring fold != fold of widened records"
    args = {k: w[k] for k in ("qkv", "decay", "beta", "slot_idx", "row_offsets",
                              "num_value_heads", "num_key_heads", "ring_slot_idx")}
    _, st_r, ring_r = oracle.recurrence_verify_ring(**args, state=w["state"], ring=ring_b0)
    _, unr_v, ring_ru = oracle.recurrence_verify_ring(**args, state=H.f32_pool(w["state"]),
                                                      ring=ring_b0)
    fold_kw = dict(slot_idx=w["slot_idx"], ring_slot_idx=w["ring_slot_idx"], accepted=acc,
                   num_value_heads=32, num_key_heads=16)
    fold_r = oracle.state_fold(state=st_r, ring=ring_r, **fold_kw)
    unr_f = oracle.state_fold(state=unr_v, ring=ring_ru, **fold_kw)
    sl = touched(w)
    ties = H.assert_state_close(fold_b[sl], fold_r[sl], "bf16-ring fold state", unr_f[sl])
    n_fit = int((lens <= ring_len).sum())
    say(f"bf16 ring: {n_fit} rows folded, fold ties {ties}")


@pytest.mark.parametrize("K", [16, 128, 256])
def test_bf16_ring_fold_multi_pass(K):
    """A bf16 ring of 19 tokens folded in several LDS passes: for every n the
    fold equals the fold of the widened float32 records bit for bit (at K = 128
    the two run different tilings: 8 and 4 columns per lane), and the full
    accepted prefixes match the oracle's bf16-ring fold within tolerance."""
    ring_len = 19
    lengths = [1, 19, 8, 20, 17]
    nk, nv = 2, 4
    w = P.small_packed(41, lengths, nk=nk, nv=nv, K=K, V=K, slots=7, state_dtype="bf16")
    stride = wl.ring_record_stride(nv // nk, K, K)
    ring0 = np.zeros((5, nk, ring_len, stride), np.uint16)
    w["ring_slot_idx"] = np.array([3, 0, 4, 1, 2], np.uint32)
    w["ring"] = ring0
    say(f"bf16 ring fold in passes: K={K} ring_len {ring_len} lengths {lengths}")
    _, st_v, ring_b = H.gpu_verify(w)
    ring_w = np.ascontiguousarray(wl.bf16_bits_to_f32(ring_b))
    for n in range(0, ring_len + 1):
        acc = np.array([min(n, L) if L <= ring_len else L for L in lengths], np.uint32)
        fold_b = H.gpu_fold(w, st_v, ring_b, acc)
        fold_w = H.gpu_fold(w, st_v, ring_w, acc)
        assert np.array_equal(fold_b, fold_w), (K, n)
    acc = np.array([L if L <= ring_len else L for L in lengths], np.uint32)
    args = {k: w[k] for k in ("qkv", "decay", "beta", "slot_idx", "row_offsets",
                              "num_value_heads", "num_key_heads", "ring_slot_idx")}
    _, st_r, ring_r = oracle.recurrence_verify_ring(**args, state=w["state"], ring=ring0)
    _, unr_v, ring_ru = oracle.recurrence_verify_ring(**args, state=H.f32_pool(w["state"]),
                                                      ring=ring0)
    fold_kw = dict(slot_idx=w["slot_idx"], ring_slot_idx=w["ring_slot_idx"], accepted=acc,
                   num_value_heads=nv, num_key_heads=nk)
    fold_r = oracle.state_fold(state=st_r, ring=ring_r, **fold_kw)
    unr_f = oracle.state_fold(state=unr_v, ring=ring_ru, **fold_kw)
    fold_g = H.gpu_fold(w, st_v, ring_b, acc)
    sl = w["slot_idx"].astype(np.int64)
    H.assert_state_close(fold_g[sl], fold_r[sl], f"bf16-ring fold K={K}", unr_f[sl])


# ------------------------------------------------------- bf16 work dtype ---

def _bits(a):
    a = np.asarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a


def _widened(w, keys):
    return dict(w, **{k: wl.bf16_bits_to_f32(w[k]) for k in keys if w.get(k) is not None})


def test_bf16_work_dtype_packed():
    """bf16 qkv / decay / beta / output (verify page, work_dtype) through the
    forward and the verify: against the oracle (outputs within tolerance or a
    bf16 rounding tie of the oracle's unrounded output), and on the GPU bit for
    bit the float32 path on the widened inputs with its output rounded once."""
    import torch
    keys = ("qkv", "decay", "beta")
    w = wl.bf16_work(wl.decode_step(batch=96, slots=128))
    ww = _widened(w, keys)
    say("bf16 work: decode step B=96")
    out_b, st_b = H.gpu_fwd(w)
    out_w, st_w = H.gpu_fwd(ww)
    assert out_b.dtype == np.uint16
    want = torch.from_numpy(out_w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out_b, want), "bf16 output != rounded float32-path output"
    assert np.array_equal(st_b, st_w)
    out_r, st_r = oracle_fwd(w)
    out_u, _ = oracle_fwd(ww)
    ties = H.assert_state_close(out_b, out_r, "bf16 work output", out_u)
    sl = touched(w)
    _, unr = oracle_fwd(w, state=H.f32_pool(w["state"]))
    ties += H.assert_state_close(st_b[sl], st_r[sl], "bf16 work state", unr[sl])
    # verify with bf16 work: output == forward output, ring == float32 path's
    v = wl.bf16_work(wl.verify_window())
    vw = _widened(v, keys)
    o_vb, s_vb, r_vb = H.gpu_verify(v)
    o_vw, s_vw, r_vw = H.gpu_verify(vw)
    o_fb, _ = H.gpu_fwd(v)
    assert np.array_equal(o_vb, o_fb), "bf16 verify output != bf16 forward output"
    assert np.array_equal(_bits(r_vb), _bits(r_vw)) and np.array_equal(s_vb, s_vw)
    want = torch.from_numpy(o_vw).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(o_vb, want)
    say(f"bf16 work packed: ties {ties}")


def test_bf16_work_dtype_fused():
    """Fused update with bf16 q, k, v, g, beta and o: GPU == float32 path on
    the widened inputs (output rounded once), and the oracle within tolerance."""
    import torch
    rng = np.random.Generator(np.random.PCG64(95))
    w = wl.bf16_work(wl.gdp_inputs(rng, B=24, S_draft=4, M=2, H=4, HV=8, K=128, V=128,
                                   slots=30, pad_frac=0.1, state_sigma=0.05))
    ww = _widened(w, ("q", "k", "v", "g", "beta"))
    say("bf16 work: fused B=24 T=8 spt=2")
    o_b, st_b, i_b = H.gpu_fused(w)
    o_w, st_w, i_w = H.gpu_fused(ww)
    assert o_b.dtype == np.uint16
    want = torch.from_numpy(o_w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(o_b, want)
    assert np.array_equal(st_b, st_w) and np.array_equal(i_b, i_w)
    o_r, st_r, _ = fused_oracle(w)
    o_u, _, _ = fused_oracle(ww)
    ties = H.assert_state_close(o_b, o_r, "bf16 work fused output", o_u)
    say(f"bf16 work fused: ties {ties}")


# ------------------------------------------------------- head dims, K != V ---

@pytest.mark.parametrize("K,V", [(256, 256), (64, 128), (128, 64), (128, 256), (256, 128)])
@pytest.mark.parametrize("S_draft", [3, 20])
def test_fused_head_dims(K, V, S_draft):
    """Fused update at the other built head dims (K != V included), short
    rows and long rows (the two launch shapes), bf16 cache with snapshots:
    against the oracle; last snapshot == final state bit for bit."""
    rng = np.random.Generator(np.random.PCG64(300 + K + V + S_draft))
    w = wl.gdp_inputs(rng, B=6, S_draft=S_draft, M=2, H=2, HV=4, K=K, V=V, slots=9,
                      pad_frac=0.2, state_sigma=0.05)
    say(f"fused head dims K={K} V={V} T={2 * S_draft}")
    o_g, st_g, inter_g = H.gpu_fused(w)
    o_r, st_r, inter_r = fused_oracle(w)
    _, st_u, inter_u = fused_oracle(w, f32=True)
    err = H.assert_close(o_g, o_r, f"K{K}V{V} output")
    idx = w["state_indices"]
    sl = idx[idx >= 0].astype(np.int64)
    ties = H.assert_state_close(st_g[sl], st_r[sl], f"K{K}V{V} state", st_u[sl])
    ties += H.assert_state_close(inter_g[sl], inter_r[sl], f"K{K}V{V} snapshots", inter_u[sl])
    assert np.array_equal(inter_g[sl, -1], st_g[sl])
    others = np.setdiff1d(np.arange(9), sl)
    assert np.array_equal(st_g[others], w["state"][others])
    say(f"K{K}V{V}: out rel err {err:.2e}, ties {ties}")


# ------------------------------------------------------ Pass-1 causal Conv1d ---

def _conv_oracle(w, silu=True, with_state=True):
    return oracle.causal_conv1d(x=w["x"], weight=w["weight"], bias=w["bias"],
                                conv_state=w["conv_state"] if with_state else None,
                                slot_idx=w["slot_idx"], row_offsets=w["row_offsets"], silu=silu)


@pytest.mark.parametrize("work", ["f32", "bf16"])
def test_conv_prefill(work):
    """Conv1d over the ragged prefill's rows (19,515 tokens x 8,192 channels,
    W = 4, history, bias, SiLU) against the oracle; the new history is the
    inputs' copy, bit for bit."""
    w = wl.conv_prefill(work_dtype=work)
    say(f"conv prefill {work}: T={w['x'].shape[0]} C=8192 W=4")
    out_g, st_g = H.gpu_conv(w)
    out_r, st_r = _conv_oracle(w)
    if work == "bf16":
        x32 = dict(w, x=wl.bf16_bits_to_f32(w["x"]), conv_state=wl.bf16_bits_to_f32(w["conv_state"]))
        out_u, _ = _conv_oracle(x32)
        ties = H.assert_state_close(out_g, out_r, "conv prefill output", out_u)
    else:
        ties = 0
        H.assert_close(out_g, out_r, "conv prefill output")
    assert np.array_equal(st_g, st_r), "conv history after the rows"
    say(f"conv prefill {work}: ties {ties}")


def test_conv_decode_and_continuity():
    """Decode shape (256 rows x 1 token) against the oracle; splitting rows
    over two calls equals one call bit for bit; zero history; padding and
    empty rows."""
    w = wl.conv_decode()
    say("conv decode B=256")
    out_g, st_g = H.gpu_conv(w)
    out_r, st_r = _conv_oracle(w)
    H.assert_close(out_g, out_r, "conv decode output")
    assert np.array_equal(st_g, st_r)
    rng = np.random.Generator(np.random.PCG64(97))
    lengths = [9, 0, 4, 17, 1, 6]
    v = wl.conv_inputs(rng, lengths, C=256, W=4, slots=8, pad_rows=(4,))
    whole, st_whole = H.gpu_conv(v)
    ref, st_ref = _conv_oracle(v)
    H.assert_close(whole, ref, "conv ragged output")
    assert np.array_equal(st_whole, st_ref)
    off = v["row_offsets"].astype(np.int64)
    cut = [3, 0, 4, 1, 1, 5]
    st_mid = None
    for part in (0, 1):
        rows = [np.arange(off[b], off[b] + cut[b]) if part == 0 else
                np.arange(off[b] + cut[b], off[b + 1]) for b in range(len(lengths))]
        o2 = np.zeros(len(lengths) + 1, np.uint32)
        o2[1:] = np.cumsum([len(r) for r in rows])
        sub = dict(v, x=np.ascontiguousarray(v["x"][np.concatenate(rows)]), row_offsets=o2,
                   conv_state=v["conv_state"] if part == 0 else st_mid)
        out_p, st_mid = H.gpu_conv(sub)
        assert np.array_equal(out_p.view(np.uint32), whole[np.concatenate(rows)].view(np.uint32))
    assert np.array_equal(st_mid, st_whole)
    z = whole[off[4]:off[5]]
    assert not z.view(np.uint32).any()
    assert np.array_equal(st_whole[v["slot_idx"][1]], v["conv_state"][v["slot_idx"][1]])
    nz, _ = H.gpu_conv(v, silu=False, with_state=False)
    nz_r, _ = _conv_oracle(v, silu=False, with_state=False)
    H.assert_close(nz, nz_r, "conv zero-history output")


@pytest.mark.parametrize("W", [2, 3, 4])
def test_conv_one_token_rows(W):
    """One-token rows update their history in the output launch: a bf16
    decode step, and one-token rows inside 8-token runs (rows of 1, 30, 1, 1,
    0, 1 tokens, one of them padding) next to longer rows; histories bit-exact
    against the oracle, untouched slots unchanged."""
    rng = np.random.Generator(np.random.PCG64(98 + W))
    d = wl.conv_inputs(rng, [1] * 64, C=512, W=W, slots=80, work_dtype="bf16")
    out_g, st_g = H.gpu_conv(d)
    out_r, st_r = _conv_oracle(d)
    x32 = dict(d, x=wl.bf16_bits_to_f32(d["x"]), conv_state=wl.bf16_bits_to_f32(d["conv_state"]))
    out_u, _ = _conv_oracle(x32)
    H.assert_state_close(out_g, out_r, f"conv bf16 decode W={W}", out_u)
    assert np.array_equal(st_g, st_r), "bf16 decode history"
    m = wl.conv_inputs(rng, [1, 30, 1, 1, 0, 1], C=256, W=W, slots=9, pad_rows=(3,))
    assert m["x"].shape[0] >= 4 * 6  # the 8-token-run launch shape
    out_g, st_g = H.gpu_conv(m)
    out_r, st_r = _conv_oracle(m)
    H.assert_close(out_g, out_r, f"conv mixed rows W={W}")
    assert np.array_equal(st_g, st_r), "mixed rows history"
    say(f"conv one-token rows W={W}: ok")


@pytest.mark.parametrize("shape", ["runs", "one_token"])
def test_conv_tokens_outside_rows(shape):
    """x holds tokens before offsets[0] and after offsets[B] (a padded token
    buffer): they belong to no row, so their output rows keep their previous
    contents and nothing is read for them; the rows themselves match the
    oracle, histories bit for bit.  Both launch shapes (8-token runs, and one
    token per thread when rows average under four tokens)."""
    rng = np.random.Generator(np.random.PCG64(131 if shape == "runs" else 132))
    if shape == "runs":
        lengths, lead, trail = [7, 0, 15, 3], 3, 21
    else:
        lengths, lead, trail = [1] * 10 + [2], 2, 9
    m = wl.conv_inputs(rng, lengths, C=128, W=4, slots=16)
    T_rows = m["x"].shape[0]
    x = rng.standard_normal((lead + T_rows + trail, 128)).astype(np.float32)
    x[lead:lead + T_rows] = m["x"]
    off = (m["row_offsets"].astype(np.int64) + lead).astype(np.uint32)
    T = x.shape[0]
    B = len(lengths)
    assert (T >= 4 * B) == (shape == "runs")
    xs = H.dev(x)
    out = torch.full((T, 128), float("nan"), device="cuda")
    st = H.dev(m["conv_state"])
    gdr.gdr_causal_conv1d(xs, H.dev(m["weight"]), H.dev(off), bias=H.dev(m["bias"]),
                          conv_state=st, slot_idx=H.dev(m["slot_idx"]), silu=True, out=out)
    torch.cuda.synchronize()
    out_g, st_g = H.host(out), H.host(st)
    out_r, st_r = oracle.causal_conv1d(x=x, weight=m["weight"], slot_idx=m["slot_idx"],
                                       row_offsets=off, bias=m["bias"],
                                       conv_state=m["conv_state"], silu=True)
    rows = slice(int(off[0]), int(off[-1]))
    H.assert_close(out_g[rows], out_r[rows], f"conv rows between padding tokens ({shape})")
    assert np.isnan(out_g[:int(off[0])]).all() and np.isnan(out_g[int(off[-1]):]).all(), (
        "tokens outside the rows were written")
    assert np.array_equal(st_g, st_r), "history"
    say(f"conv with {lead} leading and {trail} trailing tokens ({shape}): ok")


def test_debug_index_checks():
    """With gdr_set_debug_checks on, every entry point checks its device index
    vectors before enqueueing: a repeated slot, an offset past the tokens or a
    ring row out of range is rejected with nothing written, and valid calls
    give the same bits as with the checks off."""
    w = wl.verify_window()
    before = gdr.gdr_set_debug_checks(True)
    try:
        out_on, st_on, ring_on = H.gpu_verify(w)
        fold_on = H.gpu_fold(w, st_on, ring_on, w["accepted"])
        fo, fs = H.gpu_fwd(w)
        g = wl.gdp_decode()
        o_on, s_on, i_on = H.gpu_fused(g)
        bad = dict(w, slot_idx=w["slot_idx"].copy())
        bad["slot_idx"][5] = bad["slot_idx"][9]
        with pytest.raises(gdr.GdrError, match="used by rows 5 and 9"):
            H.gpu_fwd(bad)
        past = dict(w, row_offsets=w["row_offsets"].copy())
        past["row_offsets"][-1] += 1
        with pytest.raises(gdr.GdrError, match="past the"):
            H.gpu_fwd(past)
        lens = np.diff(w["row_offsets"].astype(np.int64))
        rec = int(np.flatnonzero(lens <= w["ring"].shape[2])[0])
        ring_bad = dict(w, ring_slot_idx=w["ring_slot_idx"].copy())
        ring_bad["ring_slot_idx"][rec] = w["ring"].shape[0]
        with pytest.raises(gdr.GdrError, match=f"ring row {w['ring'].shape[0]} of row {rec}"):
            H.gpu_verify(ring_bad)
        gbad = dict(g, state_indices=g["state_indices"].copy())
        act = np.flatnonzero(gbad["state_indices"] >= 0)
        gbad["state_indices"][act[1]] = gbad["state_indices"][act[0]]
        with pytest.raises(gdr.GdrError, match="used by rows"):
            H.gpu_fused(gbad)
        # a rejected call wrote nothing
        st_t = H.dev(w["state"])
        out_t = torch.full((w["qkv"].shape[0], 32 * 128), float("nan"), device="cuda")
        with pytest.raises(gdr.GdrError):
            gdr.gdr_recurrence_fwd(out_t, st_t, H.dev(bad["slot_idx"]), H.dev(w["qkv"]),
                                   H.dev(w["decay"]), H.dev(w["beta"]), H.dev(w["row_offsets"]),
                                   num_value_heads=32, num_key_heads=16)
        torch.cuda.synchronize()
        assert np.array_equal(H.host(st_t), w["state"]) and torch.isnan(out_t).all().item()
    finally:
        gdr.gdr_set_debug_checks(before)
    out_off, st_off, ring_off = H.gpu_verify(w)
    assert np.array_equal(out_on.view(np.uint32), out_off.view(np.uint32))
    assert np.array_equal(st_on, st_off) and np.array_equal(ring_on, ring_off)
    assert np.array_equal(fold_on, H.gpu_fold(w, st_off, ring_off, w["accepted"]))
    assert np.array_equal(fs, H.gpu_fwd(w)[1]) and np.array_equal(fo, H.gpu_fwd(w)[0])
    o_off, s_off, i_off = H.gpu_fused(g)
    assert np.array_equal(o_on, o_off) and np.array_equal(s_on, s_off)
    assert np.array_equal(i_on, i_off)
    say("debug index checks: rejections before launch, valid calls unchanged")


# ------------------------------------------------------------- degenerate ---

@pytest.mark.parametrize("lengths", [[200, 37, 300, 5, 64, 1], [8, 3, 1, 6, 7, 2]])
def test_extreme_decays(lengths):
    """Decays that drive the scaled state through its renormalisation: tiny
    (1e-3 and 1e-30 per token, far past 2^-64 in a few tokens), exact zeros
    mid-row, exactly 1, slightly above 1, and mixed; beta = 0 on some tokens.
    Long-row and short-row shapes against the oracle; verify == forward and
    fold(n) == forward(prefix n) bit for bit."""
    rng = np.random.Generator(np.random.PCG64(401))
    w = wl.packed_inputs(rng, lengths, nk=2, nv=4, K=128, V=128, slots=8, state_dtype="f32",
                         state_sigma=0.3)
    off = w["row_offsets"].astype(np.int64)
    patterns = [1e-3, 1e-30, 1.0, 1.01, None, 0.5]
    for b, pat in enumerate(patterns[:len(lengths)]):
        seg = slice(off[b], off[b + 1])
        if pat is None:  # zeros at every 7th token, random elsewhere
            d = w["decay"][seg]
            d[::7] = 0.0
        else:
            w["decay"][seg] = pat
    w["beta"][::5] = 0.0
    say(f"extreme decays, lengths {lengths}")
    out_g, st_g = check_fwd_against_oracle(w, f"extreme decays {lengths}")
    assert np.isfinite(out_g).all() and np.isfinite(st_g).all()
    ring_len = 8
    G, K, V = 2, 128, 128
    w["ring"] = np.zeros((8, 2, ring_len, wl.ring_record_stride(G, K, V)), np.float32)
    w["ring_slot_idx"] = np.arange(len(lengths), dtype=np.uint32)
    out_v, st_v, ring_v = H.gpu_verify(w)
    assert np.array_equal(out_v.view(np.uint32), out_g.view(np.uint32))
    lens = np.diff(off)
    acc = np.array([max(1, L // 2) if L <= ring_len else L for L in lens], np.uint32)
    folded = H.gpu_fold(w, st_v, ring_v, acc)
    keep = np.concatenate([np.arange(off[b], off[b] + acc[b]) for b in range(len(lens))])
    offs = np.zeros(len(lens) + 1, np.uint32)
    offs[1:] = np.cumsum(acc)
    _, st_pre = H.gpu_fwd(dict(w, qkv=w["qkv"][keep], decay=w["decay"][keep],
                               beta=w["beta"][keep], row_offsets=offs))
    for b in range(len(lens)):
        s = w["slot_idx"][b]
        assert np.array_equal(folded[s].view(np.uint32), st_pre[s].view(np.uint32)), b


@pytest.mark.parametrize("L", [3, 40])
def test_degenerate_tokens(L):
    """Degenerate tokens of the update, L2 norm on, on the short-row (L = 3)
    and long-row (L = 40) shapes: zero keys (k_hat = 0, so no write and
    r = 0: the state only decays), zero queries (every output 0), and a token
    with beta = 1 followed by the same key with beta = 0, a = 1 and q = k, which
    reads back exactly what was written (scale * v).  Against the oracle too."""
    nk, nv, K, V = 2, 4, 128, 128
    w = wl.packed_inputs(np.random.Generator(np.random.PCG64(420 + L)), [L, L, L], nk=nk,
                         nv=nv, K=K, V=V, slots=6, state_dtype="f32", state_sigma=0.3)
    off = w["row_offsets"].astype(np.int64)
    qc, kc = slice(0, nk * K), slice(nk * K, 2 * nk * K)
    w["qkv"][off[0]:off[1], kc] = 0.0          # row 0: zero keys
    w["qkv"][off[1]:off[2], qc] = 0.0          # row 1: zero queries
    t0 = off[2]                                # row 2: write, then read the same key back
    w["beta"][t0] = 1.0
    w["qkv"][t0 + 1, kc] = w["qkv"][t0, kc]
    w["qkv"][t0 + 1, qc] = w["qkv"][t0, kc]
    w["beta"][t0 + 1] = 0.0
    w["decay"][t0 + 1] = 1.0
    say(f"degenerate tokens, L={L}")
    out, st = check_fwd_against_oracle(w, f"degenerate tokens L={L}")
    S0 = w["state"]
    a = np.prod(w["decay"][off[0]:off[1]].astype(np.float64), axis=0)   # [nv]
    want = (a[:, None, None] * S0[w["slot_idx"][0]].astype(np.float64)).astype(np.float32)
    H.assert_close(st[w["slot_idx"][0]], want, "zero keys: the state only decays", rel=1e-5)
    assert not out[off[1]:off[2]].any(), "zero queries: every output is 0"
    sc = oracle.default_scale(K)
    v0 = w["qkv"][t0, 2 * nk * K:]
    H.assert_close(out[t0 + 1], sc * v0, "beta = 1 then the same key reads v back", rel=1e-5)


def test_large_decode_batch():
    """2048 one-token rows (8,192 workgroups) against the oracle: index
    arithmetic of large grids, every row checked."""
    rng = np.random.Generator(np.random.PCG64(402))
    w = wl.packed_inputs(rng, [1] * 2048, nk=4, nv=8, K=128, V=128, slots=4096,
                         state_dtype="bf16", state_sigma=0.05)
    say("large decode batch: 2048 rows x 8 value heads")
    check_fwd_against_oracle(w, "large decode batch")


@pytest.mark.parametrize("rows", [256, 257])
def test_longest_first_row_order(rows):
    """Ragged batches at the row-ordering limit (256 rows, 2,048 workgroups:
    workgroups take rows longest first) and one past it (index order):
    lengths with many ties,
    empty rows, lengths past the last length bucket and a padding row; every
    row against the oracle."""
    rng = np.random.Generator(np.random.PCG64(403))
    lengths = rng.choice([0, 1, 2, 3, 5, 8, 12, 13, 20, 62, 63, 64, 75], size=rows,
                         p=[.05, .2, .15, .1, .1, .1, .1, .05, .05, .03, .03, .02, .02])
    w = P.small_packed(404, lengths, nk=4, nv=8, K=128, V=128, slots=rows + 11,
                       state_dtype="bf16", sigma=0.05)
    w["slot_idx"][rows // 3] = wl.PAD_SLOT_U32
    say(f"row order: {rows} rows, {int(lengths.sum())} tokens")
    check_fwd_against_oracle(w, f"row order {rows}")


@pytest.mark.parametrize("rows", [1, 4])
def test_tiny_decode_batch(rows):
    """Decode batches small enough for the narrow-tile decode shape (1 and 4
    rows x 32 value heads): against the oracle, and bit for bit the same rows
    run inside a 64-row batch (the wide decode shape)."""
    big = wl.decode_step(seed=405, batch=64, slots=128)
    small = dict(big, qkv=big["qkv"][:rows], decay=big["decay"][:rows], beta=big["beta"][:rows],
                 slot_idx=big["slot_idx"][:rows].copy(),
                 row_offsets=big["row_offsets"][:rows + 1].copy())
    say(f"tiny decode batch: {rows} rows")
    out_s, st_s = check_fwd_against_oracle(small, f"tiny decode {rows}")
    out_b, st_b = H.gpu_fwd(big)
    assert np.array_equal(out_s.view(np.uint32), out_b[:rows].view(np.uint32)), "output bits"
    sl = small["slot_idx"].astype(np.int64)
    assert np.array_equal(st_s[sl], st_b[sl]), "state bits"


@pytest.mark.parametrize("lengths,ring_len", [
    ([1, 17, 3, 24, 2, 40, 5, 41, 9, 2, 1, 3], 40),   # short-row shape
    ([17, 40, 33, 41, 24, 16], 40),                   # long-row shape
    ([1, 2, 0, 1, 5, 1], 1),                          # a one-token ring
])
def test_records_across_stages(lengths, ring_len):
    """A ring of 40 tokens, so recorded windows span several 8- or 32-token
    stages, and a ring of one token: verify output == forward output and the
    long rows' state == forward state (bit for bit), short rows' state
    untouched, and fold(n) == forward over the first n tokens for n across
    stage boundaries."""
    nk, nv, K = 2, 4, 128
    nb = len(lengths)
    w = P.small_packed(406, lengths, nk=nk, nv=nv, K=K, V=K, slots=nb + 3, state_dtype="bf16",
                       sigma=0.05)
    w["ring"] = np.zeros((nb + 1, nk, ring_len, wl.ring_record_stride(nv // nk, K, K)),
                         np.float32)
    w["ring_slot_idx"] = np.random.Generator(np.random.PCG64(407)).permutation(nb + 1)[:nb].astype(
        np.uint32)
    say(f"records across stages: lengths {lengths}, ring_len {ring_len}")
    out_v, st_v, ring_v = H.gpu_verify(w)
    out_f, st_f = H.gpu_fwd(w)
    assert np.array_equal(out_v.view(np.uint32), out_f.view(np.uint32)), "verify output"
    out_r, _ = oracle_fwd(w)
    H.assert_close(out_v, out_r, "verify output vs oracle")
    for b, L in enumerate(lengths):
        s = w["slot_idx"][b]
        want = st_f[s] if L > ring_len else w["state"][s]
        assert np.array_equal(st_v[s], want), f"row {b} state after verify"
    off = w["row_offsets"].astype(np.int64)
    for n in (0, 1, 7, 8, 9, 16, 17, 31, 32, 33, 40):
        acc = np.array([min(n, L) if L <= ring_len else L for L in lengths], np.uint32)
        folded = H.gpu_fold(w, st_v, ring_v, acc)
        keep = np.concatenate([np.arange(off[b], off[b] + acc[b]) for b in range(nb)])
        offs = np.zeros(nb + 1, np.uint32)
        offs[1:] = np.cumsum(acc)
        _, st_pre = H.gpu_fwd(dict(w, qkv=w["qkv"][keep], decay=w["decay"][keep],
                                   beta=w["beta"][keep], row_offsets=offs))
        for b in range(nb):
            s = w["slot_idx"][b]
            assert np.array_equal(folded[s], st_pre[s]), (n, b)


def test_graph_capture_replays():
    """The decode forward and the fused GDP update captured in a HIP graph
    (torch.cuda.CUDAGraph) and replayed three times, the pool reset by eager
    copies between replays: every replay equals the eager call bit for bit."""
    import torch
    import gated_delta_rule_loop_amd as gdr
    bits = lambda x: x.view(torch.int16) if x.element_size() == 2 else x.view(torch.int32)  # noqa: E731
    w = wl.decode_step(seed=408, batch=32, slots=64)
    t = {k: H.dev(w[k]) for k in ("qkv", "decay", "beta", "state", "slot_idx", "row_offsets")}
    out = torch.empty((32, 32 * 128), device="cuda")
    gw = wl.gdp_decode(seed=409, batch=16, slots=32)
    f = {k: H.dev(gw[k]) for k in ("q", "k", "v", "g", "beta", "state", "intermediate_states")}
    f_idx = H.dev(np.asarray(gw["state_indices"], np.int32))
    o_f = torch.empty_like(f["v"])
    init = {"pool": t["state"].clone(), "gdp": f["state"].clone(),
            "snap": f["intermediate_states"].clone()}

    def reset():
        t["state"].copy_(init["pool"])
        f["state"].copy_(init["gdp"])
        f["intermediate_states"].copy_(init["snap"])
        out.zero_()
        o_f.zero_()

    def step():
        gdr.gdr_recurrence_fwd(out, t["state"], t["slot_idx"], t["qkv"], t["decay"], t["beta"],
                               t["row_offsets"], num_value_heads=32, num_key_heads=16)
        gdr.gdr_fused_recurrent_update(f["q"], f["k"], f["v"], g=f["g"], beta=f["beta"],
                                       scale=gw["scale"], use_qk_l2norm_in_kernel=True,
                                       state=f["state"], state_indices=f_idx,
                                       intermediate_states=f["intermediate_states"],
                                       steps_per_token=gw["steps_per_token"], o=o_f)

    step()
    torch.cuda.synchronize()
    eager = [bits(x).clone() for x in (out, t["state"], o_f, f["state"], f["intermediate_states"])]
    reset()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    names = ("output", "pool", "GDP output", "GDP state", "snapshots")
    for r in range(3):
        reset()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [bits(x) for x in (out, t["state"], o_f, f["state"], f["intermediate_states"])]
        for n, a, b in zip(names, got, eager):
            assert torch.equal(a, b), f"replay {r}: {n}"
    say("graph capture: 3 replays bit-identical to eager")


def _sweep_case(i):
    """Seeded random shape i: head dim, GQA, batch, length mix, pool dtype,
    ring length and ring dtype."""
    r = np.random.Generator(np.random.PCG64(5000 + i))
    K = int(r.choice([16, 32, 64, 128, 256]))
    nk = int(r.choice([1, 2, 4]))
    nv = nk * int(r.choice([1, 2, 4]))
    B = int(r.integers(1, 13))
    mix = r.choice(["decode", "short", "long", "mixed"])
    if mix == "decode":
        lengths = r.integers(0, 2, size=B)
    elif mix == "short":
        lengths = r.integers(0, 13, size=B)
    elif mix == "long":
        lengths = r.integers(16, 70, size=B)
    else:
        lengths = np.where(r.random(B) < 0.5, r.integers(0, 5, size=B), r.integers(20, 80, size=B))
    state_dtype = str(r.choice(["f32", "bf16"]))
    ring_len = int(r.choice([1, 4, 8, 16]))
    ring_bf16 = bool(r.random() < 0.5)
    return K, nk, nv, lengths.astype(np.int64), state_dtype, ring_len, ring_bf16


@pytest.mark.parametrize("i", range(64))
def test_random_shape_sweep(i):
    """64 seeded random configurations across head dims, GQA ratios, batch
    sizes, length mixes (every launch profile), pool dtypes and rings: the
    forward against the oracle; verify output == forward output bit for bit
    and against the oracle; ring records against the oracle's; the fold
    against the oracle, and (float32 ring) == forward over the prefix."""
    K, nk, nv, lengths, sd, ring_len, ring_bf16 = _sweep_case(i)
    B = len(lengths)
    say(f"sweep {i}: K={K} nk={nk} nv={nv} lengths={lengths.tolist()} pool={sd} "
        f"ring_len={ring_len} ring_bf16={ring_bf16}")
    w = P.small_packed(6000 + i, lengths, nk=nk, nv=nv, K=K, V=K, slots=B + 4, state_dtype=sd,
                       sigma=0.05)
    out_f, st_f = check_fwd_against_oracle(w, f"sweep {i} fwd")
    ring_dt = np.uint16 if ring_bf16 else np.float32
    w["ring"] = np.zeros((B + 2, nk, ring_len, wl.ring_record_stride(nv // nk, K, K)), ring_dt)
    w["ring_slot_idx"] = np.random.Generator(np.random.PCG64(7000 + i)).permutation(B + 2)[:B].astype(
        np.uint32)
    out_v, st_v, ring_v = H.gpu_verify(w)
    assert np.array_equal(out_v.view(np.uint32), out_f.view(np.uint32)), "verify output bits"
    out_r, st_r, ring_r = verify_oracle(w)
    H.assert_close(out_v, out_r, f"sweep {i} verify output")
    ring_unr = None
    if ring_bf16:  # unrounded records: the oracle with a float32 ring
        ring_unr = verify_oracle(dict(w, ring=np.zeros(w["ring"].shape, np.float32)))[2]
    H.assert_state_close(ring_v, ring_r, f"sweep {i} ring records", ring_unr)
    for b, L in enumerate(lengths):
        s = w["slot_idx"][b]
        want = st_f[s] if L > ring_len else w["state"][s]
        assert np.array_equal(st_v[s], want), f"row {b} state after verify"
    acc = np.array([L // 2 + 1 if 0 < L <= ring_len else L for L in lengths], np.uint32)
    acc = np.minimum(acc, lengths).astype(np.uint32)
    folded = H.gpu_fold(w, st_v, ring_v, acc)
    fold_r = oracle.state_fold(state=st_v, slot_idx=w["slot_idx"], ring=ring_v,
                               ring_slot_idx=w["ring_slot_idx"], accepted=acc,
                               num_value_heads=nv, num_key_heads=nk)
    sl = w["slot_idx"].astype(np.int64)
    fold_unr = None
    if sd == "bf16":  # unrounded fold: the oracle on a float32 copy of the pool
        fold_unr = oracle.state_fold(state=H.f32_pool(st_v), slot_idx=w["slot_idx"], ring=ring_v,
                                     ring_slot_idx=w["ring_slot_idx"], accepted=acc,
                                     num_value_heads=nv, num_key_heads=nk)[sl]
    H.assert_state_close(folded[sl], fold_r[sl], f"sweep {i} fold", fold_unr)
    if not ring_bf16:
        off = w["row_offsets"].astype(np.int64)
        keep = np.concatenate([np.arange(off[b], off[b] + acc[b]) for b in range(B)])
        offs = np.zeros(B + 1, np.uint32)
        offs[1:] = np.cumsum(acc)
        _, st_pre = H.gpu_fwd(dict(w, qkv=w["qkv"][keep], decay=w["decay"][keep],
                                   beta=w["beta"][keep], row_offsets=offs))
        assert np.array_equal(folded[sl], st_pre[sl]), "fold == forward prefix"


_FUSED_DIMS = [(16, 16), (32, 32), (64, 64), (128, 128), (256, 256), (64, 128), (128, 64),
               (128, 256), (256, 128)]


@pytest.mark.parametrize("i", range(48))
def test_random_fused_sweep(i):
    """48 seeded random fused updates: head dims (K != V included), GQA,
    batch, draft and copy counts (steps_per_token), padding, pool dtype,
    per-column or head-wise or absent beta, absent log decay, and inputs with
    or without the DeltaProduct structure: output, pool and snapshots against
    the oracle; last snapshot == final state; untouched slots unchanged."""
    r = np.random.Generator(np.random.PCG64(8000 + i))
    K, V = _FUSED_DIMS[int(r.integers(len(_FUSED_DIMS)))]
    Hh = int(r.choice([1, 2, 4]))
    HV = Hh * int(r.choice([1, 2]))
    Bn, S_draft, M = int(r.integers(1, 9)), int(r.integers(1, 12)), int(r.choice([1, 2, 3]))
    sd = str(r.choice(["f32", "bf16"]))
    slots = Bn + 3
    w = wl.gdp_inputs(r, B=Bn, S_draft=S_draft, M=M, H=Hh, HV=HV, K=K, V=V, slots=slots,
                      pad_frac=float(r.choice([0.0, 0.3])), state_sigma=0.05, state_dtype=sd,
                      beta_per_v=bool(r.random() < 0.3))
    if r.random() < 0.5:  # general inputs: query and decay on every step
        w["q"] = r.standard_normal(w["q"].shape).astype(np.float32)
        w["g"] = (-np.logaddexp(0.0, r.standard_normal(w["g"].shape))).astype(np.float32)
    if r.random() < 0.2:
        w["g"] = None
    if r.random() < 0.2:
        w["beta"] = None
    say(f"fused sweep {i}: K={K} V={V} H={Hh} HV={HV} B={Bn} T={S_draft * M} spt={M} pool={sd} "
        f"beta={'none' if w['beta'] is None else w['beta'].ndim} g={'none' if w['g'] is None else 'yes'}")
    o_g, st_g, inter_g = H.gpu_fused(w)
    o_r, st_r, inter_r = fused_oracle(w)
    _, st_u, inter_u = fused_oracle(w, f32=True) if sd == "bf16" else (None, None, None)
    H.assert_close(o_g, o_r, f"fused sweep {i} output")
    idx = np.asarray(w["state_indices"])
    sl = idx[idx >= 0].astype(np.int64)
    pad = idx < 0
    assert not o_g[pad].view(np.uint32).any(), "padding rows' output"
    H.assert_state_close(st_g[sl], st_r[sl], f"fused sweep {i} state",
                         None if st_u is None else st_u[sl])
    H.assert_state_close(inter_g[sl], inter_r[sl], f"fused sweep {i} snapshots",
                         None if inter_u is None else inter_u[sl])
    assert np.array_equal(inter_g[sl, -1], st_g[sl]), "last snapshot == final state"
    others = np.setdiff1d(np.arange(slots), sl)
    assert np.array_equal(st_g[others], w["state"][others])
    assert np.array_equal(inter_g[others].view(np.uint8), w["intermediate_states"][others].view(np.uint8))


@pytest.mark.parametrize("i", range(32))
def test_random_conv_sweep(i):
    """32 seeded random Conv1d calls: channel counts (multiples of 4, a
    partial last workgroup included), widths 2-4, f32 and bf16, ragged lengths
    with empty and one-token rows on both launch shapes, padding rows, bias or
    none, SiLU or none, with or without history: output against the oracle,
    history bit for bit."""
    r = np.random.Generator(np.random.PCG64(9000 + i))
    C = int(r.choice([4, 12, 64, 260, 1028]))
    W = int(r.choice([2, 3, 4]))
    work = str(r.choice(["f32", "bf16"]))
    Bn = int(r.integers(1, 10))
    lengths = (r.integers(0, 3, size=Bn) if r.random() < 0.5 else r.integers(0, 30, size=Bn))
    pads = tuple(int(b) for b in np.flatnonzero(r.random(Bn) < 0.2))
    w = wl.conv_inputs(r, lengths, C=C, W=W, slots=Bn + 2, work_dtype=work, pad_rows=pads)
    if r.random() < 0.3:
        w["bias"] = None
    silu, with_state = bool(r.random() < 0.7), bool(r.random() < 0.8)
    say(f"conv sweep {i}: C={C} W={W} {work} lengths={lengths.tolist()} pads={pads} "
        f"bias={w['bias'] is not None} silu={silu} state={with_state}")
    out_g, st_g = H.gpu_conv(w, silu=silu, with_state=with_state)
    out_r, st_r = _conv_oracle(w, silu=silu, with_state=with_state)
    if work == "bf16":
        x32 = dict(w, x=wl.bf16_bits_to_f32(w["x"]), conv_state=wl.bf16_bits_to_f32(w["conv_state"]))
        out_u, _ = _conv_oracle(x32, silu=silu, with_state=with_state)
        H.assert_state_close(out_g, out_r, f"conv sweep {i} output", out_u)
    else:
        H.assert_close(out_g, out_r, f"conv sweep {i} output")
    if with_state:
        assert np.array_equal(st_g, st_r), "history"


def test_all_rows_empty():
    """Batches whose rows are all empty (zero tokens, so the per-token tensors
    have no elements and torch hands over null pointers): every entry point
    accepts them and leaves the pools, ring and histories unchanged."""
    import torch
    import gated_delta_rule_loop_amd as gdr
    w = P.small_packed(410, [0, 0, 0], nk=2, nv=4, K=128, V=128, slots=5, state_dtype="bf16")
    w["slot_idx"][1] = wl.PAD_SLOT_U32
    assert w["qkv"].shape[0] == 0
    out_g, st_g = H.gpu_fwd(w)
    assert out_g.shape == (0, 512) and np.array_equal(st_g, w["state"])
    w["ring"] = np.zeros((4, 2, 8, wl.ring_record_stride(2, 128, 128)), np.float32)
    w["ring_slot_idx"] = np.array([3, 0, 2], np.uint32)
    _, st_v, ring_v = H.gpu_verify(w)
    assert np.array_equal(st_v, w["state"]) and not ring_v.any()
    folded = H.gpu_fold(w, st_v, ring_v, np.zeros(3, np.uint32))
    assert np.array_equal(folded, w["state"])
    g = wl.gdp_inputs(np.random.Generator(np.random.PCG64(411)), B=1, S_draft=1, M=1, H=2, HV=4,
                      K=128, V=128, slots=4, pad_frac=0.0, state_sigma=0.05)
    q = torch.empty((1, 0, 2, 128), device="cuda")
    v = torch.empty((1, 0, 4, 128), device="cuda")
    gl = torch.empty((1, 0, 4), device="cuda")
    st = H.dev(g["state"])
    cu = torch.zeros(4, dtype=torch.int32, device="cuda")  # three empty sequences
    idx = torch.tensor([2, -1, 0], dtype=torch.int32, device="cuda")
    o, _ = gdr.gdr_fused_recurrent_update(q, q, v, g=gl, beta=gl, cu_seqlens=cu, state=st,
                                          state_indices=idx, use_qk_l2norm_in_kernel=True)
    torch.cuda.synchronize()
    assert o.shape == (1, 0, 4, 128) and np.array_equal(H.host(st), g["state"])
    c = wl.conv_inputs(np.random.Generator(np.random.PCG64(412)), [0, 0], C=64, W=4, slots=3)
    out_c, st_c = H.gpu_conv(c)
    assert out_c.shape == (0, 64) and np.array_equal(st_c, c["conv_state"])
    say("all rows empty: every entry point a no-op")


@pytest.mark.parametrize("i", range(24))
def test_random_rollback_sweep(i):
    """24 seeded random rollbacks: every built K, V pair, both pool dtypes,
    1-6 snapshots, accepted counts in [0, I+1], padding, indices and counts
    as i32 or u32: the pool bit for bit against the oracle's copy."""
    import torch
    import gated_delta_rule_loop_amd as gdr
    r = np.random.Generator(np.random.PCG64(9500 + i))
    K, V = _FUSED_DIMS[int(r.integers(len(_FUSED_DIMS)))]
    HV, I, N = int(r.choice([1, 2, 8])), int(r.integers(1, 7)), int(r.integers(1, 20))
    S = N + 4
    sd = str(r.choice(["f32", "bf16"]))
    draw = lambda shape: r.standard_normal(shape).astype(np.float32)  # noqa: E731
    state = draw((S, HV, K, V))
    inter = draw((S, I, HV, K, V))
    if sd == "bf16":
        state, inter = wl.to_bf16_bits(state), wl.to_bf16_bits(inter)
    idx = r.permutation(S)[:N].astype(np.int32)
    idx[r.random(N) < 0.2] = -1
    acc = r.integers(0, I + 2, size=N).astype(np.int32)
    as_u32 = bool(r.random() < 0.5)
    say(f"rollback sweep {i}: K={K} V={V} HV={HV} I={I} N={N} {sd} u32={as_u32}")
    st_t = H.dev(state)
    conv = (lambda a: H.dev(a.view(np.uint32))) if as_u32 else (lambda a: H.dev(a))  # noqa: E731
    gdr.gdr_snapshot_rollback(st_t, conv(idx), H.dev(inter), conv(acc))
    torch.cuda.synchronize()
    want = oracle.snapshot_rollback(state=state, state_indices=idx, intermediate_states=inter,
                                    accepted=acc)
    assert np.array_equal(H.host(st_t).view(np.uint8), want.view(np.uint8))


@pytest.mark.parametrize("i", range(32))
def test_random_bf16_work_sweep(i):
    """32 seeded random shapes (as the shape sweep) with bf16 per-token inputs
    and outputs: forward and verify bit for bit the float32 path on the
    widened inputs with the output rounded once (state and ring records equal),
    and the forward output against the oracle (tolerance or rounding tie)."""
    import torch
    K, nk, nv, lengths, sd, ring_len, ring_bf16 = _sweep_case(100 + i)
    B = len(lengths)
    say(f"bf16 work sweep {i}: K={K} nk={nk} nv={nv} lengths={lengths.tolist()} pool={sd}")
    keys = ("qkv", "decay", "beta")
    w = wl.bf16_work(P.small_packed(6500 + i, lengths, nk=nk, nv=nv, K=K, V=K, slots=B + 4,
                                    state_dtype=sd, sigma=0.05))
    ww = _widened(w, keys)
    rnd = lambda a: torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)  # noqa: E731
    out_b, st_b = H.gpu_fwd(w)
    out_w, st_w = H.gpu_fwd(ww)
    assert np.array_equal(out_b, rnd(out_w)) and np.array_equal(st_b, st_w), "forward"
    out_r, _ = oracle_fwd(w)
    out_u, _ = oracle_fwd(ww)
    H.assert_state_close(out_b, out_r, f"bf16 work sweep {i} output", out_u)
    ring_dt = np.uint16 if ring_bf16 else np.float32
    for d in (w, ww):
        d["ring"] = np.zeros((B + 2, nk, ring_len, wl.ring_record_stride(nv // nk, K, K)), ring_dt)
        d["ring_slot_idx"] = np.arange(B, dtype=np.uint32)[::-1].copy()
    o_vb, s_vb, r_vb = H.gpu_verify(w)
    o_vw, s_vw, r_vw = H.gpu_verify(ww)
    assert np.array_equal(o_vb, out_b), "verify output == forward output"
    assert np.array_equal(o_vb, rnd(o_vw)) and np.array_equal(s_vb, s_vw), "verify"
    assert np.array_equal(_bits(r_vb), _bits(r_vw)), "ring records"


def test_element_offsets_past_2_to_31():
    """Maximum-size indexing: 6,000 rows of 1,000 tokens with one key and one
    value head at K = V = 128 and bf16 per-token tensors, so qkv holds 2.3e9
    elements and the last rows start past element 2^31 (byte offsets past
    2^32).  Every row gets the same inputs and the same initial state, so every
    row must give the same output and final-state bits; the last row is also
    checked against the oracle."""
    import torch

    import gated_delta_rule_loop_amd as gdr
    rows, L = 6000, 1000
    base = wl.bf16_work(P.small_packed(8800, [L], nk=1, nv=1, K=128, V=128, slots=1,
                                       state_dtype="f32", sigma=0.05))
    conv = base["qkv"].shape[1]
    assert (rows - 1) * L * conv > 2**31
    say(f"offsets past 2^31: {rows} rows x {L} tokens, qkv [{rows * L}, {conv}] bf16")
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(  # noqa: E731
        torch.bfloat16).cuda()
    qkv = bf(base["qkv"]).repeat(rows, 1)
    decay = bf(base["decay"]).repeat(rows, 1)
    beta = bf(base["beta"]).repeat(rows, 1)
    state = torch.from_numpy(base["state"]).cuda().repeat(rows, 1, 1, 1)
    slots = torch.arange(rows, dtype=torch.int32, device="cuda")
    offs = torch.arange(rows + 1, dtype=torch.int32, device="cuda") * L
    out = torch.full((rows * L, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    gdr.gdr_recurrence_fwd(out, state, slots, qkv, decay, beta, offs, num_value_heads=1,
                           num_key_heads=1)
    torch.cuda.synchronize()
    ob = out.view(torch.int16).view(rows, L * 128)
    sb = state.view(torch.int32).view(rows, -1)
    assert bool((ob == ob[:1]).all()), "every row's output bits equal row 0's"
    assert bool((sb == sb[:1]).all()), "every row's final state equals row 0's"
    del qkv, decay, beta
    last_out = ob[-1].cpu().numpy().view(np.uint16).reshape(L, 128)
    last_state = state[-1:].cpu().numpy()
    out_r, st_r = oracle_fwd(base)
    out_u, _ = oracle_fwd(_widened(base, ("qkv", "decay", "beta")))
    H.assert_state_close(last_out, out_r, "last row output (bf16)", out_u)
    H.assert_close(last_state, st_r, "last row final state")
    say("offsets past 2^31: all rows bit-identical, last row within tolerance of the oracle")


def test_conv_element_offsets_past_2_to_31():
    """Maximum-size indexing for the Conv1d: 6,000 rows of 1,000 tokens at
    C = 384 in bf16 (2.3e9 elements of x; the last rows start past element
    2^31), every row with the same inputs and history: all rows' outputs and
    new histories bit-identical, the last row against the oracle (history bit
    for bit)."""
    import torch

    import gated_delta_rule_loop_amd as gdr
    rows, L, C, W = 6000, 1000, 384, 4
    base = wl.conv_inputs(np.random.Generator(np.random.PCG64(8810)), [L], C=C, W=W, slots=1,
                          work_dtype="bf16")
    base["slot_idx"] = np.zeros(1, np.uint32)
    assert (rows - 1) * L * C > 2**31
    say(f"conv offsets past 2^31: {rows} rows x {L} tokens x {C} channels, bf16")
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(  # noqa: E731
        torch.bfloat16).cuda()
    x = bf(base["x"]).repeat(rows, 1)
    hist = bf(base["conv_state"]).repeat(rows, 1, 1)
    weight = torch.from_numpy(base["weight"]).cuda()
    bias = torch.from_numpy(base["bias"]).cuda()
    slots = torch.arange(rows, dtype=torch.int32, device="cuda")
    offs = torch.arange(rows + 1, dtype=torch.int32, device="cuda") * L
    out = gdr.gdr_causal_conv1d(x, weight, offs, bias=bias, conv_state=hist, slot_idx=slots,
                                silu=True)
    torch.cuda.synchronize()
    del x
    ob = out.view(torch.int16).view(rows, L * C)
    hb = hist.view(torch.int16).view(rows, -1)
    assert bool((ob == ob[:1]).all()), "every row's output bits equal row 0's"
    assert bool((hb == hb[:1]).all()), "every row's new history equals row 0's"
    last_out = ob[-1].cpu().numpy().view(np.uint16).reshape(L, C)
    last_hist = hb[-1:].cpu().numpy().view(np.uint16).reshape(1, W - 1, C)
    out_r, st_r = _conv_oracle(base, silu=True, with_state=True)
    x32 = dict(base, x=wl.bf16_bits_to_f32(base["x"]),
               conv_state=wl.bf16_bits_to_f32(base["conv_state"]))
    out_u, _ = _conv_oracle(x32, silu=True, with_state=True)
    H.assert_state_close(last_out, out_r, "conv last row output (bf16)", out_u)
    assert np.array_equal(last_hist, st_r), "conv last row history"
    say("conv offsets past 2^31: all rows bit-identical, last row against the oracle")


def test_fused_element_offsets_past_2_to_31():
    """Maximum-size indexing for the fused update: 6,000 requests of 1,000
    steps, H = 1, HV = 4, K = V = 128, bf16 work, so v and o hold 3.1e9
    elements and the last requests start past element 2^31.  Every request has
    the same inputs and cached state: all outputs and final states bit-identical,
    the last request against the oracle."""
    import torch

    import gated_delta_rule_loop_amd as gdr
    rows, T, HV = 6000, 1000, 4
    base = wl.bf16_work(wl.gdp_inputs(np.random.Generator(np.random.PCG64(8820)), B=1,
                                      S_draft=T, M=1, H=1, HV=HV, K=128, V=128, slots=1,
                                      pad_frac=0.0, state_sigma=0.05, state_dtype="f32"))
    base["state_indices"] = np.zeros(1, np.int32)
    base["intermediate_states"] = None
    assert (rows - 1) * T * HV * 128 > 2**31
    say(f"fused offsets past 2^31: {rows} requests x {T} steps, v [{rows}, {T}, {HV}, 128] bf16")
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(  # noqa: E731
        torch.bfloat16).cuda()
    rep = lambda t: t.repeat(rows, *([1] * (t.dim() - 1)))  # noqa: E731
    q, k, v = rep(bf(base["q"])), rep(bf(base["k"])), rep(bf(base["v"]))
    g, beta = rep(bf(base["g"])), rep(bf(base["beta"]))
    state = rep(torch.from_numpy(base["state"]).cuda())
    idx = torch.arange(rows, dtype=torch.int32, device="cuda")
    o, _ = gdr.gdr_fused_recurrent_update(q, k, v, g=g, beta=beta, scale=base["scale"],
                                          use_qk_l2norm_in_kernel=True, state=state,
                                          state_indices=idx)
    torch.cuda.synchronize()
    del q, k, v, g, beta
    ob = o.view(torch.int16).view(rows, -1)
    sb = state.view(torch.int32).view(rows, -1)
    assert bool((ob == ob[:1]).all()), "every request's output bits equal request 0's"
    assert bool((sb == sb[:1]).all()), "every request's final state equals request 0's"
    last_o = ob[-1].cpu().numpy().view(np.uint16).reshape(1, T, HV, 128)
    last_state = state[-1:].cpu().numpy()
    o_r, st_r, _ = oracle.fused_recurrent_update(**base)
    wide = _widened(base, ("q", "k", "v", "g", "beta"))
    o_u, _, _ = oracle.fused_recurrent_update(**wide)
    H.assert_state_close(last_o, o_r, "fused last request output (bf16)", o_u)
    H.assert_close(last_state, st_r, "fused last request final state")
    say("fused offsets past 2^31: all requests bit-identical, last request against the oracle")
