"""Benchmark of the gated delta rule recurrence on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--only decode,decode_bf16,prefill,verify,verify_bf16ring,gdp,
                            gdp_v256,gdp_betacols,conv,decode_small]
                    [--no-cpu-baseline] [--copy-probe MiB] [--verify-window L]

Headline: the decode step (256 sequences x 1 token, nk=16, nv=32, K=V=128,
bf16 state pool of 512 slots) through gdr_recurrence_fwd; `value` is decode
tokens/s with every input already resident in HBM.  Cold-cache protocol: R
independent sets of (pool, inputs, outputs) are rotated so that consecutive
launches touch disjoint memory (R * 512 MiB of pool, well above the 256 MB
Infinity Cache).  The per-launch time is the HIP-event time of the timed
region on the stream the kernels run on, divided by the launch count.

Also timed (reported under "configs"): the decode step with bf16 per-token
inputs and output, the ragged prefill (VALU-bound), the speculative verify +
fold with a float32 and with a bf16 ring (HBM-bound), the Gated DeltaProduct
decode with snapshots and the snapshot rollback (HBM-bound), and that decode
with V = 256 (K != V) and with per-column beta; the Pass-1 causal Conv1d over
the prefill's rows and over a decode step (HBM-bound); decode steps of 1, 4,
16 and 64 sequences.  Each case also reports single-launch p10 / median / p90
and the mean single launch of each rotation set.

The CPU baseline is the plain C oracle timed on the host on whole decode
batches, once on N threads (its independent (sequence, value head) items
farmed over the host's cores; `cores` = N) and once on one thread
(`threads_1`), with the CPU model from /proc/cpuinfo.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
VALU_FP32_PEAK_TFLOPS = 78.6     # 256 CU x 4 SIMD x 16 lanes x 2 (FMA) x 2.4 GHz, unpacked
VALU_FP32_PACKED_TFLOPS = 157.3  # with packed fp32 (not used by these kernels)
FLOPS_PER_TOKEN_HEAD_ELEM = 7    # decay 1, S^T k 2, rank-1 write 2, S^T q 2 per state element


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("gdr_device.h", "gdr_kernels.hip", "gdr_rec_table.hip", "gdr_api.cpp",
              "gdr_internal.h", "gdr_fastdiv.h"):
        with open(os.path.join(ROOT, "gated_delta_rule_loop_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(case):
    """HBM traffic per launch measured with rocprofv3 counters, if the summary
    in profiles/ was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{case}.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"^traffic-json: (\{.*\})$", open(path).read(), flags=re.M)
    if not m:
        return None
    d = json.loads(m.group(1))
    if d.get("kernel_hash") != kernel_source_hash():
        return None
    return d


# ------------------------------------------------------------------ cases ---

class Case:
    """One timed workload: R rotation sets and a launch for each."""

    def __init__(self, name, launches, alg_bytes, state_bytes, tokens, flops=0.0, extra=None):
        self.name = name
        self.launches = launches
        self.alg_bytes = alg_bytes
        self.state_bytes = state_bytes
        self.tokens = tokens
        self.flops = flops
        self.extra = extra or {}


def _dev(torch, a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.int32)).cuda()
    return torch.from_numpy(a).cuda()


def _packed_launch(torch, gdr, B, w, ring=False, stream=None):
    """Prebuilt C-ABI call of the forward (or verify) on device copies of w."""
    d = {k: _dev(torch, w[k]) for k in ("qkv", "decay", "beta", "state", "slot_idx",
                                       "row_offsets")}
    T = w["qkv"].shape[0]
    V = w["state"].shape[3]
    work = torch.bfloat16 if w["qkv"].dtype == np.uint16 else torch.float32
    d["out"] = torch.empty((T, w["num_value_heads"] * V), dtype=work, device="cuda")
    keep = dict(d)
    L = B.lib()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    descs = [B.describe(d[k]) for k in ("out", "state", "slot_idx", "qkv", "decay", "beta",
                                        "row_offsets")]
    refs = [ctypes.byref(x) for x in descs]
    nv, nk = w["num_value_heads"], w["num_key_heads"]
    if ring:
        keep["ring"] = _dev(torch, w["ring"])
        keep["ring_slot_idx"] = _dev(torch, w["ring_slot_idx"])
        rdesc = [B.describe(keep["ring"]), B.describe(keep["ring_slot_idx"])]
        refs += [ctypes.byref(x) for x in rdesc]
        descs += rdesc

        def launch():
            rc = L.gdr_recurrence_verify_ring(nv, nk, *refs, ctypes.c_float(-1.0), 1, st)
            assert rc == 0, B.gdr_last_error_message()
    else:
        def launch():
            rc = L.gdr_recurrence_fwd(nv, nk, *refs, ctypes.c_float(-1.0), 1, st)
            assert rc == 0, B.gdr_last_error_message()
    launch.keep = (keep, descs, refs)
    return launch, keep


def case_decode(torch, gdr, B, wl, rotations):
    launches = []
    for r in range(rotations):
        w = wl.decode_step(seed=1001 + 100 * r)
        launch, _ = _packed_launch(torch, gdr, B, w)
        launches.append(launch)
    Bn, nv, K = 256, 32, 128
    state = Bn * nv * K * K * 2 * 2
    alg = state + Bn * 8192 * 4 + Bn * nv * K * 4 + 2 * Bn * nv * 4 + (2 * Bn + 1) * 4
    flops = FLOPS_PER_TOKEN_HEAD_ELEM * Bn * nv * K * K
    return Case("decode_256x1", launches, alg, state, Bn, flops)


def case_decode_small(torch, gdr, B, wl, rotations, Bn):
    """A decode step of Bn one-token rows (small batches: 1, 4, 16, 64), as
    the 256-row step otherwise.  Event timing of back-to-back launches this
    short includes the host's launch cost; the kernel trace gives the device
    time."""
    launches = []
    for r in range(rotations):
        w = wl.decode_step(seed=1001 + 100 * r, batch=Bn)
        launch, _ = _packed_launch(torch, gdr, B, w)
        launches.append(launch)
    nv, K = 32, 128
    state = Bn * nv * K * K * 2 * 2
    alg = state + Bn * 8192 * 4 + Bn * nv * K * 4 + 2 * Bn * nv * 4 + (2 * Bn + 1) * 4
    flops = FLOPS_PER_TOKEN_HEAD_ELEM * Bn * nv * K * K
    return Case(f"decode_{Bn}x1", launches, alg, state, Bn, flops)


def case_decode_bf16(torch, gdr, B, wl, rotations):
    """The decode step with bf16 per-token inputs and output (work dtype)."""
    launches = []
    for r in range(rotations):
        w = wl.bf16_work(wl.decode_step(seed=1001 + 100 * r))
        launch, _ = _packed_launch(torch, gdr, B, w)
        launches.append(launch)
    Bn, nv, K = 256, 32, 128
    state = Bn * nv * K * K * 2 * 2
    alg = state + Bn * 8192 * 2 + Bn * nv * K * 2 + 2 * Bn * nv * 2 + (2 * Bn + 1) * 4
    flops = FLOPS_PER_TOKEN_HEAD_ELEM * Bn * nv * K * K
    return Case("decode_256x1_bf16io", launches, alg, state, Bn, flops)


def case_conv(torch, gdr, B, wl, rotations, decode):
    """The Pass-1 causal Conv1d (W = 4, bias, SiLU, history) over the prefill's
    rows or over a decode step's 256 one-token rows; float32 io."""
    launches = []
    for r in range(rotations):
        w = (wl.conv_decode(seed=1006 + 100 * r) if decode
             else wl.conv_prefill(seed=1005 + 100 * r))
        t = {k: _dev(torch, w[k]) for k in ("x", "weight", "bias", "conv_state", "slot_idx",
                                           "row_offsets")}
        t["out"] = torch.empty_like(t["x"])
        ds = [B.describe(t[k]) for k in ("out", "x", "weight", "bias", "conv_state", "slot_idx",
                                         "row_offsets")]
        refs = [ctypes.byref(d) for d in ds]
        L = B.lib()
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

        def launch(refs=refs, st=st, keep=(t, ds)):
            rc = L.gdr_causal_conv1d(*refs, B.GDR_FLAG_CONV_SILU, st)
            assert rc == 0, B.gdr_last_error_message()
        launches.append(launch)
    T, C = w["x"].shape
    rows = len(w["slot_idx"])
    hist = rows * 3 * C * 4 * 2
    alg = 2 * T * C * 4 + hist + C * 5 * 4
    name = "conv_decode_256x1" if decode else "conv_prefill_8x4096"
    return Case(name, launches, alg, hist, T, 2 * 4 * T * C)


def case_prefill(torch, gdr, B, wl, rotations):
    w = wl.ragged_prefill()
    launches = []
    for r in range(rotations):
        launch, _ = _packed_launch(torch, gdr, B, w)
        launches.append(launch)
    T = w["qkv"].shape[0]
    lens = np.diff(w["row_offsets"].astype(np.int64))
    nv, K = 32, 128
    state = 8 * nv * K * K * 2 * 2
    alg = state + w["qkv"].nbytes + T * nv * K * 4 + 2 * T * nv * 4
    flops = FLOPS_PER_TOKEN_HEAD_ELEM * T * nv * K * K
    return Case("prefill_8x4096", launches, alg, state, T, flops,
                extra={"max_len": int(lens.max()), "lengths": lens.tolist()})


def case_verify_fold(torch, gdr, B, wl, rotations, ring_bf16=False, fixed_len=None):
    w = wl.verify_window(fixed_len=fixed_len)
    suffix = "" if fixed_len is None else f"_len{fixed_len}"
    if ring_bf16:  # the same window with a bf16 ring (verify page, ring_dtype)
        w = dict(w, ring=np.zeros(w["ring"].shape, np.uint16))
        suffix += "_bf16ring"
    ring_es = 2 if ring_bf16 else 4
    lens = np.diff(w["row_offsets"].astype(np.int64))
    ring_len = w["ring"].shape[2]
    verifies, folds = [], []
    for r in range(rotations):
        launch, keep = _packed_launch(torch, gdr, B, w, ring=True)
        verifies.append(launch)
        acc = _dev(torch, w["accepted"])
        ds = [B.describe(x) for x in (keep["state"], keep["slot_idx"], keep["ring"],
                                      keep["ring_slot_idx"], acc)]
        refs = [ctypes.byref(x) for x in ds]
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        L = B.lib()

        def fold(refs=refs, st=st, keepalive=(acc, ds, keep)):
            rc = L.gdr_state_fold(32, 16, *refs, st)
            assert rc == 0, B.gdr_last_error_message()
        folds.append(fold)
    nv, nk, K, V, G = 32, 16, 128, 128, 2
    head = K * V * 2
    rec = K + G * (V + 1)
    T = int(lens.sum())
    long_rows = lens > ring_len
    state_v = 64 * nv * head + int(long_rows.sum()) * nv * head
    ring_w = int(lens[~long_rows].sum()) * nk * rec * ring_es
    alg_v = state_v + ring_w + w["qkv"].nbytes + T * nv * V * 4 + 2 * T * nv * 4
    acc = w["accepted"].astype(np.int64)
    fold_rows = (acc > 0) & (acc <= ring_len)
    state_f = int(fold_rows.sum()) * nv * head * 2
    alg_f = state_f + int(acc[fold_rows].sum()) * nk * rec * ring_es
    cv = Case("verify_64x12" + suffix, verifies, alg_v, state_v + ring_w, T,
              FLOPS_PER_TOKEN_HEAD_ELEM * T * nv * K * V,
              extra={"long_rows": int(long_rows.sum())})
    cf = Case("fold_64x12" + suffix, folds, alg_f, state_f, int(acc[fold_rows].sum()),
              2 * 2 * int(acc[fold_rows].sum()) * nv * K * V,
              extra={"folded_rows": int(fold_rows.sum())})
    return cv, cf


def case_gdp(torch, gdr, B, wl, rotations, V=128, beta_cols=False):
    """GDP decode (B=128, 4 drafts x 2 copies, H=16, HV=32, K=128) and the
    rollback after it; variants: value head dim V (K != V) or per-column beta
    (those return the decode case only)."""
    launches = []
    rb_sets = []
    w0 = None
    variant = V != 128 or beta_cols
    for r in range(rotations):
        if variant:
            rng = np.random.Generator(np.random.PCG64(1004 + 100 * r))
            w = wl.gdp_inputs(rng, B=128, S_draft=4, M=2, H=16, HV=32, K=128, V=V, slots=160,
                              pad_frac=0.1, state_sigma=0.05, beta_per_v=beta_cols)
        else:
            w = wl.gdp_decode(seed=1004 + 100 * r)
        w0 = w0 or w
        t = {k: _dev(torch, w[k]) for k in ("q", "k", "v", "g", "beta", "state",
                                           "intermediate_states")}
        t["idx"] = _dev(torch, w["state_indices"].astype(np.int32))
        t["o"] = torch.empty(w["v"].shape, dtype=torch.float32, device="cuda")
        ds = {k: B.describe(v) for k, v in t.items()}
        L = B.lib()
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        r_ = ctypes.byref
        args = (r_(ds["q"]), r_(ds["k"]), r_(ds["v"]), r_(ds["g"]), r_(ds["beta"]),
                ctypes.c_float(-1.0), None, None, 1, None, r_(ds["state"]), r_(ds["idx"]),
                r_(ds["intermediate_states"]), 2, r_(ds["o"]), st)

        def launch(args=args, keep=(t, ds)):
            rc = L.gdr_fused_recurrent_update(*args)
            assert rc == 0, B.gdr_last_error_message()
        launches.append(launch)
        rb_sets.append((t, ds, L))
    idx = w0["state_indices"]
    act = int((idx >= 0).sum())
    # rollback after verification: request n accepts (n mod 5) draft tokens
    acc = np.resize(np.arange(5, dtype=np.int32), len(idx))
    rb_launches = []
    for t, ds, L_ in rb_sets:
        a_t = _dev(torch, acc)
        a_d = B.describe(a_t)
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        rargs = (ctypes.byref(ds["state"]), ctypes.byref(ds["idx"]),
                 ctypes.byref(ds["intermediate_states"]), ctypes.byref(a_d), st)

        def rollback(rargs=rargs, keep=(t, ds, a_t, a_d)):
            rc = L_.gdr_snapshot_rollback(*rargs)
            assert rc == 0, B.gdr_last_error_message()
        rb_launches.append(rollback)
    rolled = int(((idx >= 0) & (acc >= 1) & (acc <= 4)).sum())
    HV, H, K, T = 32, 16, 128, 8
    head = K * V * 2
    state = act * HV * head * 2 + act * HV * head * (T // 2)
    beta_elems = HV * V if beta_cols else HV
    inputs = act * T * (2 * H * K + HV * V + HV + beta_elems) * 4
    outs = 128 * T * HV * V * 4
    name = "gdp_128x8" + (f"_K128V{V}" if V != 128 else "") + ("_betacols" if beta_cols else "")
    gdp = Case(name, launches, state + inputs + outs, state, act * T,
               FLOPS_PER_TOKEN_HEAD_ELEM * act * T * HV * K * V,
               extra={"active_rows": act, "draft_tokens": act * T // 2})
    if variant:
        return (gdp,)
    rb_bytes = rolled * HV * head * 2
    rb = Case("rollback_128x4", rb_launches, rb_bytes, rb_bytes, rolled,
              extra={"rolled_rows": rolled})
    return gdp, rb


# ----------------------------------------------------------------- timing ---

def time_case(torch, case, steps, warmup):
    stream = torch.cuda.current_stream()
    n = len(case.launches)
    for i in range(warmup):
        case.launches[i % n]()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        case.launches[i % n]()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end)
    return ms / steps, wall


def launch_spread(torch, case, n):
    """p10 / median / p90 of single launches (one HIP event pair around each, on
    the launch stream), taken after the timed region, and the mean single
    launch of each rotation set (the spread across buffer sets); the reported
    rate comes from the back-to-back timed region, not from these."""
    stream = torch.cuda.current_stream()
    m = len(case.launches)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for i, (a, b) in enumerate(ev):
        a.record(stream)
        case.launches[i % m]()
        b.record(stream)
    torch.cuda.synchronize()
    times = [a.elapsed_time(b) * 1e3 for a, b in ev]
    by_set = [round(float(np.mean(times[j::m])), 2) for j in range(min(m, n))]
    us = sorted(times)
    return [round(us[n // 10], 2), round(us[n // 2], 2), round(us[(9 * n) // 10], 2)], by_set


def summarize(case, ms_per_launch):
    s = ms_per_launch * 1e-3
    d = {"us_per_launch": round(ms_per_launch * 1e3, 2),
         "tokens_per_s": round(case.tokens / s, 1),
         "alg_bytes_per_launch": int(case.alg_bytes),
         "alg_GBps": round(case.alg_bytes / s / 1e9, 1),
         "state_GBps": round(case.state_bytes / s / 1e9, 1),
         "hbm_frac": round(case.alg_bytes / s / 1e9 / HBM_PEAK_GBS, 4)}
    if case.flops:
        tf = case.flops / s / 1e12
        d["alg_TFLOPs"] = round(tf, 2)
        d["valu_frac_unpacked"] = round(tf / VALU_FP32_PEAK_TFLOPS, 4)
        d["valu_frac_packed_peak"] = round(tf / VALU_FP32_PACKED_TFLOPS, 4)
    d.update(case.extra)
    return d


def cpu_model():
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(wl, budget_s=5.0):
    """The oracle as it stands, on whole decode batches (256 sequences x 32
    value heads, K=V=128, bf16 pool): once on one thread, once with its
    independent (row, value head) items spread over N threads.  Only the
    oracle's own work is timed (it updates a resident copy of the pool in
    place); each leg repeats whole batches for about budget_s seconds and
    reports the median batch."""
    import oracle
    n_threads = oracle.default_threads()
    w = wl.decode_step()
    state = w["state"].copy()
    out = np.zeros((w["qkv"].shape[0], w["num_value_heads"] * w["state"].shape[3]), np.float32)
    args = {k: w[k] for k in ("qkv", "decay", "beta", "slot_idx", "row_offsets",
                              "num_value_heads", "num_key_heads")}
    tokens = w["qkv"].shape[0]
    state_bytes = 2 * tokens * w["num_value_heads"] * w["state"].shape[2] * w["state"].shape[3] * 2

    def leg(threads):
        times = []
        while sum(times) < budget_s and len(times) < 200:
            t0 = time.perf_counter()
            oracle.recurrence_fwd_into(out=out, state=state, threads=threads, **args)
            times.append(time.perf_counter() - t0)
        return float(np.median(times)), len(times)

    med1, reps1 = leg(1)
    medn, repsn = leg(n_threads)
    return {"value": round(tokens / medn, 1), "unit": "tokens/s", "cores": n_threads,
            "kind": "oracle",
            "sample": f"whole decode batches (256 sequences x 32 value heads, K=V=128, bf16 "
                      f"pool), median of {repsn} batches on {n_threads} threads and of {reps1} "
                      f"on 1 thread; the oracle's (row, value head) items farmed over the "
                      f"threads, pool updated in place",
            "cpu_model": cpu_model(),
            "state_GBps": round(state_bytes / medn / 1e9, 3),
            "threads_1": {"value": round(tokens / med1, 1), "unit": "tokens/s",
                          "state_GBps": round(state_bytes / med1 / 1e9, 3)}}


def copy_probe(torch, mib):
    """A plain device copy of known size, for calibrating the HBM counters."""
    x = torch.empty(mib * 1024 * 1024, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    x.fill_(1)
    torch.cuda.synchronize()
    for _ in range(5):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": x.numel(), "launches": 5}))


def copy_rate(torch, mib=1024, n=20):
    """Read + write GB/s of a plain 1 GiB device-to-device copy (torch's copy
    kernel), timed like the cases: the box's achievable-bandwidth reference."""
    x = torch.empty(mib * 1024 * 1024, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    x.fill_(1)
    y.copy_(x)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(n):
        y.copy_(x)
    e1.record(st)
    torch.cuda.synchronize()
    rate = 2 * x.numel() * n / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del x, y
    torch.cuda.empty_cache()
    return rate


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rotations", type=int, default=4)
    ap.add_argument("--only", default="decode,decode_bf16,prefill,verify,verify_bf16ring,gdp,"
                                      "gdp_v256,gdp_betacols,conv,decode_small")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0)
    ap.add_argument("--verify-window", type=int, default=0,
                    help="with --only verify: every window of this length (1-12) instead of "
                         "uniform in [1, 12]")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one MI355X: every (sequence, value head) recurrence is "
              "independent and has no cross-GPU step; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_loop_amd as gdr
    from gated_delta_rule_loop_amd import _binding as B
    from gated_delta_rule_loop_amd import workloads as wl

    if args.copy_probe:
        copy_probe(torch, args.copy_probe)
        return
    B.lib()
    only = set(args.only.split(","))
    cases = []
    if "decode" in only:
        cases.append(case_decode(torch, gdr, B, wl, args.rotations))
    if "decode_bf16" in only:
        cases.append(case_decode_bf16(torch, gdr, B, wl, args.rotations))
    if "prefill" in only:
        cases.append(case_prefill(torch, gdr, B, wl, 2))
    if "verify" in only:
        cases.extend(case_verify_fold(torch, gdr, B, wl, args.rotations,
                                      fixed_len=args.verify_window or None))
    if "conv" in only:
        cases.append(case_conv(torch, gdr, B, wl, args.rotations, decode=True))
        cases.append(case_conv(torch, gdr, B, wl, 2, decode=False))
    if "verify_bf16ring" in only:
        cases.extend(case_verify_fold(torch, gdr, B, wl, args.rotations, ring_bf16=True))
    if "gdp" in only:
        cases.extend(case_gdp(torch, gdr, B, wl, 2))
    if "gdp_v256" in only:
        cases.extend(case_gdp(torch, gdr, B, wl, 2, V=256))
    if "gdp_betacols" in only:
        cases.extend(case_gdp(torch, gdr, B, wl, 2, beta_cols=True))
    if "decode_small" in only:
        for Bn in (1, 4, 16, 64):
            cases.append(case_decode_small(torch, gdr, B, wl, args.rotations, Bn))
    torch.cuda.synchronize()

    results = {}
    head = None
    for c in cases:
        steps = args.steps if c.name != "prefill_8x4096" else max(5, args.steps // 40)
        ms, wall = time_case(torch, c, steps, args.warmup if c.name != "prefill_8x4096" else 2)
        results[c.name] = summarize(c, ms)
        results[c.name]["launches_timed"] = steps
        if "max_len" in results[c.name]:  # the token-serial critical path of the longest row
            results[c.name]["ns_per_step_of_longest_row"] = round(
                ms * 1e6 / results[c.name]["max_len"], 1)
        spread, by_set = launch_spread(torch, c, min(steps, 100 if c.name != "prefill_8x4096" else 5))
        results[c.name]["single_launch_us_p10_p50_p90"] = spread
        results[c.name]["single_launch_us_mean_by_set"] = by_set
        print(f"# {c.name}: {json.dumps(results[c.name])}", file=sys.stderr, flush=True)
        if c.name == "decode_256x1":
            head = (c, ms, steps)

    line = {"metric": "decode tokens/sec and achieved state HBM GB/s (% peak), 1 MI355X",
            "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": "synthetic", "configs": results}
    if head is not None:
        c, ms, steps = head
        s = ms * 1e-3
        line.update({"value": round(c.tokens / s, 1), "ms_per_step": round(ms, 5),
                     "config": {"workload": "decode step: 256 sequences x 1 token, nk=16 key "
                                            "heads, nv=32 value heads, K=V=128, bf16 state "
                                            "pool of 512 slots, f32 inputs",
                                "batch": 256, "tokens_per_sequence": 1,
                                "state_dtype": "bf16", "cold_cache_rotations": args.rotations},
                     "state_GBps": results["decode_256x1"]["state_GBps"]})
        tr = read_traffic("rec_kernel_decode_256x1tok")
        line["roofline"] = {"bound": "hbm", "achieved": round(c.alg_bytes / s / 1e9, 1),
                            "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(c.alg_bytes / s / 1e9 / HBM_PEAK_GBS, 4),
                            "traffic": None if tr is None else tr["bytes_per_launch"]}
        cp = copy_rate(torch)
        line["copy_reference"] = {"kind": "torch device copy of 1 GiB, read + write bytes",
                                  "GBps": round(cp, 1),
                                  "decode_frac_of_copy": round(c.alg_bytes / s / 1e9 / cp, 4)}
    else:
        line.update({"value": None, "ms_per_step": None, "config": {"workload": args.only}})
    if not args.no_cpu_baseline and "decode" in only:
        line["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
