"""Seeded synthetic inputs for the gated delta rule recurrence.

This module only draws inputs; it holds none of the recurrence's arithmetic.
The tests (HIP library and CPU oracle alike) and the benchmark take their
inputs from here.  Arrays are NumPy; bfloat16 tensors are carried as uint16
bit patterns (rounded to nearest even by torch's own conversion).

Workload shapes follow the operations' documented layouts:
  * packed forward / verify ("gated_delta_recurrence_fwd_gpu",
    "gated_delta_recurrence_verify_ring_gpu" Args): qkv [T, 2*nk*K + nv*V],
    decay and beta [T, nv], state pool [slots, nv, K, V], slot_idx [B],
    row offsets [B+1]; ring [rows, nk, ring_len, record_stride];
  * fused update ("core.ssm.ops.gdp.fused_recurrent" parameters):
    q, k [B, T, H, K], v [B, T, HV, V], g and beta [B, T, HV], state
    [S, HV, K, V], state_indices [B] (-1 = padding), intermediate_states
    [S, T // steps_per_token, HV, K, V].

Recipes (one NumPy PCG64 generator per workload with a fixed default seed;
normals drawn in float64, then cast):
  q, k, v ~ N(0, 1); decay a = exp(-softplus(z)); beta = sigmoid(z');
  log decay g = -softplus(z); state ~ N(0, sigma) then rounded to the pool
  dtype; slots are distinct random subsets of the pool.
"""
from __future__ import annotations

import numpy as np
import torch

PAD_SLOT_U32 = 0xFFFFFFFF


def _softplus(z):
    return np.logaddexp(0.0, z)


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float -> bfloat16 bit patterns (uint16), round to nearest even."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact widening)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


WORK_KEYS = ("qkv", "decay", "beta", "q", "k", "v", "g")


def bf16_work(w: dict) -> dict:
    """The same workload with its per-token inputs (qkv, decay, beta, or q, k,
    v, g, beta) rounded to bfloat16, as uint16 bits."""
    out = dict(w)
    for key in WORK_KEYS:
        a = out.get(key)
        if a is not None and a.dtype == np.float32:
            out[key] = to_bf16_bits(a)
    return out


def ring_record_stride(group: int, K: int, V: int, align: int = 32) -> int:
    """A record stride of at least K + group*(V+1) elements, rounded up."""
    need = K + group * (V + 1)
    return (need + align - 1) // align * align


def packed_inputs(rng, lengths, nk, nv, K, V, slots, state_dtype, state_sigma,
                  pad_rows=()):
    """Inputs of the packed forward for the given row lengths."""
    lengths = np.asarray(lengths, dtype=np.int64)
    B = len(lengths)
    T = int(lengths.sum())
    offsets = np.zeros(B + 1, dtype=np.uint32)
    offsets[1:] = np.cumsum(lengths)
    conv_dim = 2 * nk * K + nv * V
    qkv = rng.standard_normal((T, conv_dim)).astype(np.float32)
    decay = np.exp(-_softplus(rng.standard_normal((T, nv)))).astype(np.float32)
    beta = _sigmoid(rng.standard_normal((T, nv))).astype(np.float32)
    state_f = rng.standard_normal((slots, nv, K, V)) * state_sigma
    state = to_bf16_bits(state_f) if state_dtype == "bf16" else state_f.astype(np.float32)
    slot_idx = rng.choice(slots, size=B, replace=False).astype(np.uint32)
    for r in pad_rows:
        slot_idx[r] = PAD_SLOT_U32
    return dict(qkv=qkv, decay=decay, beta=beta, state=state, slot_idx=slot_idx,
                row_offsets=offsets, num_value_heads=nv, num_key_heads=nk)


def tiny_ragged(seed: int = 1000):
    """Tiny ragged forward: B=2, lengths [3,5], nk=1, nv=2, K=V=16, float32
    pool of 4 slots (std 0.1), slot_idx [3,1], scale 1/4, L2 norm on."""
    rng = np.random.Generator(np.random.PCG64(seed))
    w = packed_inputs(rng, [3, 5], nk=1, nv=2, K=16, V=16, slots=4, state_dtype="f32",
                      state_sigma=0.1)
    w["slot_idx"] = np.array([3, 1], dtype=np.uint32)
    w["scale"] = 0.25
    return w


def decode_step(seed: int = 1001, batch: int = 256, slots: int = 512):
    """Decode step: 256 sequences of one token, nk=16, nv=32, K=V=128, bf16
    pool of 512 slots (std 0.05), distinct random slots."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return packed_inputs(rng, [1] * batch, nk=16, nv=32, K=128, V=128, slots=slots,
                         state_dtype="bf16", state_sigma=0.05)


def ragged_prefill(seed: int = 1002, batch: int = 8, max_len: int = 4096, slots: int = 64):
    """Ragged prefill: 8 rows, lengths uniform in [1, 4096], heads as the
    decode step, bf16 pool of 64 slots (std 0.05), state in place."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = rng.integers(1, max_len + 1, size=batch)
    return packed_inputs(rng, lengths, nk=16, nv=32, K=128, V=128, slots=slots,
                         state_dtype="bf16", state_sigma=0.05)


def verify_window(seed: int = 1003, batch: int = 64, max_window: int = 12, ring_len: int = 8,
                  slots: int = 128, fixed_len: int | None = None):
    """Speculative verify plus fold: 64 rows with windows uniform in [1, 12],
    ring_len 8, float32 ring and bf16 pool of 128 slots each; the accepted
    count is uniform in [0, len] for rows that fit the ring and the full
    length for rows that do not (those rows commit during verify).  With
    fixed_len every window has that length (instruction-count fits)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = rng.integers(1, max_window + 1, size=batch)
    if fixed_len is not None:
        lengths = np.full(batch, fixed_len, dtype=lengths.dtype)
    w = packed_inputs(rng, lengths, nk=16, nv=32, K=128, V=128, slots=slots,
                      state_dtype="bf16", state_sigma=0.05)
    group = 32 // 16
    stride = ring_record_stride(group, 128, 128)
    w["ring"] = np.zeros((slots, 16, ring_len, stride), dtype=np.float32)
    w["ring_slot_idx"] = rng.choice(slots, size=batch, replace=False).astype(np.uint32)
    acc = np.array([rng.integers(0, n + 1) if n <= ring_len else n for n in lengths],
                   dtype=np.uint32)
    w["accepted"] = acc
    return w


def gdp_inputs(rng, B, S_draft, M, H, HV, K, V, slots, pad_frac, state_sigma,
               state_dtype="bf16", beta_per_v=False):
    """Gated DeltaProduct decode folded into the fused update: each of the
    S_draft draft tokens becomes M Householder copies; the query sits on the
    last copy (zero elsewhere) and the decay on the first (g = 0, i.e. a = 1,
    elsewhere).  beta_per_v draws one beta per value column ([B, T, HV, V]).
    Returns the fused-update inputs with steps_per_token = M."""
    T = S_draft * M
    q = rng.standard_normal((B, T, H, K)).astype(np.float32)
    k = rng.standard_normal((B, T, H, K)).astype(np.float32)
    v = rng.standard_normal((B, T, HV, V)).astype(np.float32)
    g = (-_softplus(rng.standard_normal((B, T, HV)))).astype(np.float32)
    beta_shape = (B, T, HV, V) if beta_per_v else (B, T, HV)
    beta = _sigmoid(rng.standard_normal(beta_shape)).astype(np.float32)
    copy = np.arange(T) % M
    q[:, copy != M - 1] = 0.0
    g[:, copy != 0] = 0.0
    state_f = rng.standard_normal((slots, HV, K, V)) * state_sigma
    state = to_bf16_bits(state_f) if state_dtype == "bf16" else state_f.astype(np.float32)
    idx = rng.choice(slots, size=B, replace=False).astype(np.int32)
    n_pad = int(round(pad_frac * B))
    if n_pad:
        idx[rng.choice(B, size=n_pad, replace=False)] = -1
    inter_shape = (slots, T // M, HV, K, V)
    # sentinel-filled so that untouched entries are recognisable
    if state_dtype == "bf16":
        inter = np.full(inter_shape, 0x7FC1, dtype=np.uint16)
    else:
        inter = np.full(inter_shape, np.nan, dtype=np.float32)
    return dict(q=q, k=k, v=v, g=g, beta=beta, state=state, state_indices=idx,
                intermediate_states=inter, steps_per_token=M, use_qk_l2norm_in_kernel=True,
                scale=K ** -0.5)


def gdp_decode(seed: int = 1004, batch: int = 128, slots: int = 256):
    """GDP decode: M=2 copies x S=4 drafts (T=8, steps_per_token=2), B=128 with
    10% padding, H=16, HV=32, K=V=128, bf16 state of 256 slots, intermediate
    buffer [256, 4, 32, 128, 128]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return gdp_inputs(rng, B=batch, S_draft=4, M=2, H=16, HV=32, K=128, V=128, slots=slots,
                      pad_frac=0.1, state_sigma=0.05)


def conv_inputs(rng, lengths, C, W, slots, work_dtype="f32", pad_rows=()):
    """Inputs of the Pass-1 causal Conv1d over ragged rows: x ~ N(0, 1)
    [T, C], weight ~ N(0, 1/W) [C, W], bias ~ N(0, 0.1) [C], history
    conv_state ~ N(0, 1) [slots, W-1, C] (x's dtype), distinct slots."""
    lengths = np.asarray(lengths, dtype=np.int64)
    T = int(lengths.sum())
    off = np.zeros(len(lengths) + 1, dtype=np.uint32)
    off[1:] = np.cumsum(lengths)
    x = rng.standard_normal((T, C)).astype(np.float32)
    weight = (rng.standard_normal((C, W)) / np.sqrt(W)).astype(np.float32)
    bias = (rng.standard_normal(C) * 0.1).astype(np.float32)
    state = rng.standard_normal((slots, W - 1, C)).astype(np.float32)
    slot_idx = rng.choice(slots, size=len(lengths), replace=False).astype(np.uint32)
    for r in pad_rows:
        slot_idx[r] = PAD_SLOT_U32
    if work_dtype == "bf16":
        x, state = to_bf16_bits(x), to_bf16_bits(state)
    return dict(x=x, weight=weight, bias=bias, conv_state=state, slot_idx=slot_idx,
                row_offsets=off)


def conv_prefill(seed: int = 1005, work_dtype="f32"):
    """Conv1d before the ragged prefill: the prefill's row lengths (8 rows in
    [1, 4096]), C = 2*16*128 + 32*128 = 8192 channels, W = 4, 64 slots."""
    lengths = np.random.Generator(np.random.PCG64(1002)).integers(1, 4097, size=8)
    rng = np.random.Generator(np.random.PCG64(seed))
    return conv_inputs(rng, lengths, C=8192, W=4, slots=64, work_dtype=work_dtype)


def conv_decode(seed: int = 1006, batch: int = 256, work_dtype="f32"):
    """Conv1d before a decode step: 256 rows of one token, C = 8192, W = 4,
    512 history slots."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return conv_inputs(rng, [1] * batch, C=8192, W=4, slots=512, work_dtype=work_dtype)


WORKLOADS = {"tiny_ragged": tiny_ragged, "decode_step": decode_step,
             "ragged_prefill": ragged_prefill, "verify_window": verify_window,
             "gdp_decode": gdp_decode, "conv_prefill": conv_prefill,
             "conv_decode": conv_decode}
