"""Plant plausible mistakes in copies of the oracle and check that each one
trips at least one pin (CPU only; the real oracle is never modified)."""
import os
import subprocess
import tempfile

import pytest

import oracle
from oracle import build as oracle_build
from tests import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdr_oracle.c")

# The decay and the retrieval of one step, as written in the oracle (for the
# mutation that retrieves from the undecayed state).
_DECAY = """    for (int i = 0; i < K; ++i)
        for (int j = 0; j < V; ++j)
            S[i * V + j] = a * S[i * V + j];
"""
_RETRIEVAL = """    for (int j = 0; j < V; ++j) {
        float r = 0.0f;
        for (int i = 0; i < K; ++i)
            r = r + S[i * V + j] * khat[i];
        float b = beta_per_v ? beta[j] : beta[0];
        u[j] = b * (v[j] - r);
    }
"""

# (name, original text, planted text)
MUTATIONS = [
    ("delta_sign", "u[j] = b * (v[j] - r);", "u[j] = b * (v[j] + r);"),
    ("beta_on_r_only", "u[j] = b * (v[j] - r);", "u[j] = v[j] - b * r;"),
    ("no_decay", "S[i * V + j] = a * S[i * V + j];", "S[i * V + j] = S[i * V + j];"),
    ("retrieval_transposed", "r = r + S[i * V + j] * khat[i];", "r = r + S[j * V + i] * khat[i];"),
    ("readout_with_k", "acc = acc + S[i * V + j] * qhat[i];", "acc = acc + S[i * V + j] * khat[i];"),
    ("write_v_not_u", "S[i * V + j] = S[i * V + j] + khat[i] * u[j];",
     "S[i * V + j] = S[i * V + j] + khat[i] * v[j];"),
    ("no_scale", "o[j] = scale * acc;", "o[j] = acc;"),
    ("gqa_modulo", "const int h = hv / G;", "const int h = hv % nk;"),
    ("norm_no_sqrt", "float rho = 1.0f / sqrtf(sq + ORACLE_L2NORM_EPS);",
     "float rho = 1.0f / (sq + ORACLE_L2NORM_EPS);"),
    ("bf16_truncate", "x += 0x7fffu + keep_lsb;", "x += 0u * keep_lsb;"),
    ("fold_wrong_head_a", "oracle_ring_get(ring, ring_bf16, rec + K + (int64_t)G * V + m);",
     "oracle_ring_get(ring, ring_bf16, rec + K + (int64_t)G * V);"),
    ("snapshot_off_by_one", "const int64_t i = step / steps_per_token - 1;",
     "const int64_t i = step / steps_per_token;"),
    ("padding_not_zero", "o[(f * HV + hv) * V + j] = 0.0f;", "o[(f * HV + hv) * V + j] = 1.0f;"),
    ("long_row_not_committed", "if (t1 > t0 && !use_ring)", "if (t1 > t0 && ring == NULL)"),
    ("rollback_off_by_one", "((int64_t)idx * int_tokens + (a - 1)) * block",
     "((int64_t)idx * int_tokens + a - (a > 1)) * block"),
    ("per_v_beta_ignored", "float b = beta_per_v ? beta[j] : beta[0];", "float b = beta[0];"),
    ("ring_bf16_read_truncated", "return ring_bf16 ? oracle_bf16_widen(((const uint16_t*)ring)[i])",
     "return ring_bf16 ? oracle_bf16_widen(((const uint16_t*)ring)[i] & 0xFF80u)"),
    ("conv_taps_reversed", "y = y + weight[(int64_t)c * W + j] * window[j];",
     "y = y + weight[(int64_t)c * W + (W - 1 - j)] * window[j];"),
    ("conv_history_reversed", "conv_state[((int64_t)slot * H + i) * C + c] = hist[i];",
     "conv_state[((int64_t)slot * H + i) * C + c] = hist[H - 1 - i];"),
    ("conv_silu_sign", "y = y / (1.0f + expf(-y));", "y = y / (1.0f + expf(y));"),
    ("offsets_shifted", "const int64_t t0 = row_offsets[b], t1 = row_offsets[b + 1];",
     "const int64_t t0 = row_offsets[b] + (b > 0), t1 = row_offsets[b + 1];"),
    ("readout_before_write", "acc = acc + S[i * V + j] * qhat[i];",
     "acc = acc + (S[i * V + j] - khat[i] * u[j]) * qhat[i];"),
    ("retrieval_before_decay", _DECAY + "\n" + _RETRIEVAL, _RETRIEVAL + "\n" + _DECAY),
    ("q_not_normalised", "        oracle_l2norm(K, q, qhat);\n",
     "        for (int i = 0; i < K; ++i)\n            qhat[i] = q[i];\n"),
    ("log_decay_not_exponentiated", "const float a = g ? expf(g[f * HV + hv]) : 1.0f;",
     "const float a = g ? g[f * HV + hv] : 1.0f;"),
    ("fold_u_of_head_0", "rec + K + (int64_t)m * V + j", "rec + K + j"),
    ("snapshot_step_not_sequence_local", "const int64_t step = f - f0 + 1;",
     "const int64_t step = f + 1;"),
    ("initial_state_ignored",
     "oracle_load_block(initial_state, state_bf16, ((int64_t)n * HV + hv) * kv, kv, S);",
     "for (int64_t e = 0; e < kv; ++e) S[e] = 0.0f;"),
    ("conv_history_ignored",
     "window[j] = conv_state[((int64_t)slot * H + (H + (s - t0))) * C + c];",
     "window[j] = 0.0f;"),
    ("conv_short_row_drops_old_history",
     "hist[i] = conv_state[((int64_t)slot * H + (L + i)) * C + c];", "hist[i] = 0.0f;"),
    ("conv_bias_dropped",
     "float y = bias ? bias[c] : 0.0f;", "float y = 0.0f;"),
]


@pytest.mark.parametrize("name,orig,planted", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, orig, planted, tmp_path):
    with open(SRC) as f:
        text = f.read()
    assert orig in text, f"mutation site for {name} no longer exists in the oracle"
    mutant = os.path.join(tmp_path, f"{name}.c")
    with open(mutant, "w") as f:
        f.write(text.replace(orig, planted, 1))  # first site: the step itself
    lib = os.path.join(tmp_path, f"lib{name}.so")
    subprocess.run(["gcc", *oracle_build.CFLAGS, mutant, "-o", lib, "-lm"], check=True)
    failed = []
    with oracle.using_library(lib):
        for pin in oracle_pins.ALL_PINS:
            try:
                pin()
            except (AssertionError, ValueError):
                failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {name}"
