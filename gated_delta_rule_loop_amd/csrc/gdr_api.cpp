// Host side of the C ABI declared in include/gdr.h: argument validation,
// launch-shape choice and dispatch to the gfx950 kernels.  Nothing here
// allocates, frees or synchronises device memory, except the optional index
// checks (gdr_set_debug_checks), which copy index vectors to the host.
#include "gdr.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <utility>
#include <vector>

#include "gdr_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

bool present(const gdr_tensor* t) { return t != nullptr && t->data != nullptr; }

const char* dtype_name(int32_t d) {
    switch (d) {
        case GDR_DTYPE_F32: return "f32";
        case GDR_DTYPE_BF16: return "bf16";
        case GDR_DTYPE_U32: return "u32";
        case GDR_DTYPE_I32: return "i32";
        default: return "?";
    }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Rank, dtype and exact shape check; a shape entry < 0 matches anything.
// A tensor with a zero extent: its data pointer may be null (an allocator's
// empty buffer), and nothing is read or written through it.
bool empty(const gdr_tensor* t) {
    if (t->ndim < 1 || t->ndim > 5) return false;
    for (int i = 0; i < t->ndim; ++i)
        if (t->shape[i] == 0) return true;
    return false;
}

// A required tensor that is missing (an empty one may have a null pointer).
bool missing(const gdr_tensor* t) { return t == nullptr || (t->data == nullptr && !empty(t)); }

int check_tensor(const char* fn, const char* name, const gdr_tensor* t, int ndim,
                 const int64_t* shape, bool allow_f32, bool allow_bf16, bool allow_idx) {
    if (missing(t)) return fail(GDR_ERR_INVALID_ARG, "%s: %s is null", fn, name);
    if (t->ndim != ndim)
        return fail(GDR_ERR_INVALID_ARG, "%s: %s must have rank %d (got %d)", fn, name, ndim,
                    t->ndim);
    const bool ok = (allow_f32 && t->dtype == GDR_DTYPE_F32) ||
                    (allow_bf16 && t->dtype == GDR_DTYPE_BF16) ||
                    (allow_idx && (t->dtype == GDR_DTYPE_U32 || t->dtype == GDR_DTYPE_I32));
    if (!ok)
        return fail(GDR_ERR_UNSUPPORTED, "%s: %s has unsupported dtype %s", fn, name,
                    dtype_name(t->dtype));
    for (int i = 0; i < ndim; ++i) {
        if (t->shape[i] < 0)
            return fail(GDR_ERR_INVALID_ARG, "%s: %s has a negative extent", fn, name);
        if (shape && shape[i] >= 0 && t->shape[i] != shape[i])
            return fail(GDR_ERR_INVALID_ARG, "%s: %s dim %d is %lld, expected %lld", fn, name, i,
                        static_cast<long long>(t->shape[i]), static_cast<long long>(shape[i]));
    }
    return GDR_OK;
}

// Innermost stride 1, 16-byte base, outer strides multiples of `mult`.
int check_layout(const char* fn, const char* name, const gdr_tensor* t, int64_t mult) {
    if (empty(t)) return GDR_OK;  // nothing is read or written through it
    if (t->stride[t->ndim - 1] != 1)
        return fail(GDR_ERR_UNSUPPORTED, "%s: %s must have unit innermost stride", fn, name);
    if (!aligned16(t->data))
        return fail(GDR_ERR_UNSUPPORTED, "%s: %s base must be 16-byte aligned", fn, name);
    for (int i = 0; i < t->ndim - 1; ++i)
        if (t->stride[i] % mult != 0)
            return fail(GDR_ERR_UNSUPPORTED, "%s: %s stride %d must be a multiple of %lld", fn,
                        name, i, static_cast<long long>(mult));
    return GDR_OK;
}

int check_index_vec(const char* fn, const char* name, const gdr_tensor* t, int64_t n) {
    const int64_t shape[1] = {n};
    int rc = check_tensor(fn, name, t, 1, shape, false, false, true);
    if (rc) return rc;
    if (n > 1 && t->stride[0] != 1)
        return fail(GDR_ERR_UNSUPPORTED, "%s: %s must be contiguous", fn, name);
    return GDR_OK;
}

// Every per-token tensor of a call shares the work dtype (f32 or bf16).
int check_work_dtype(const char* fn, const char* name, const gdr_tensor* t, int32_t work) {
    if (present(t) && t->dtype != work)
        return fail(GDR_ERR_UNSUPPORTED, "%s: %s is %s but the work dtype is %s", fn, name,
                    dtype_name(t->dtype), dtype_name(work));
    return GDR_OK;
}

// Outer-stride multiple (in elements) that keeps 16-byte rows for a dtype.
int64_t vec_mult(int32_t dtype) { return dtype == GDR_DTYPE_BF16 ? 8 : 4; }

bool head_dim_built(int64_t K) {
    return K == 16 || K == 32 || K == 64 || K == 128 || K == 256;
}

// Key/value head dims with kernels: K == V in 16..256, and for the fused
// update (K != V) the pairs below.
bool dims_built(int64_t K, int64_t V, bool allow_kv_differ) {
    if (K == V) return head_dim_built(K);
    if (!allow_kv_differ) return false;
    return (K == 64 && V == 128) || (K == 128 && V == 64) || (K == 128 && V == 256) ||
           (K == 256 && V == 128);
}
const char* kDimsBuilt = "K == V in {16, 32, 64, 128, 256}; fused update also (K, V) in "
                         "{(64, 128), (128, 64), (128, 256), (256, 128)}";

// State-like tensor [slots, nv, K, V] with a dense K x V block per head.
int check_state(const char* fn, const char* name, const gdr_tensor* t, int ndim,
                const int64_t* shape, bool allow_kv_differ = false) {
    int rc = check_tensor(fn, name, t, ndim, shape, true, true, false);
    if (rc) return rc;
    const int64_t K = t->shape[ndim - 2], V = t->shape[ndim - 1];
    if (K != V && !allow_kv_differ)
        return fail(GDR_ERR_UNSUPPORTED, "%s: %s needs K == V", fn, name);
    if (!dims_built(K, V, allow_kv_differ))
        return fail(GDR_ERR_UNSUPPORTED, "%s: head dims K=%lld V=%lld not built (%s)", fn,
                    static_cast<long long>(K), static_cast<long long>(V), kDimsBuilt);
    if (!empty(t) && (t->stride[ndim - 1] != 1 || t->stride[ndim - 2] != V))
        return fail(GDR_ERR_UNSUPPORTED, "%s: %s needs a dense K x V block per head", fn, name);
    return check_layout(fn, name, t, t->dtype == GDR_DTYPE_BF16 ? 8 : 4);
}

// ------------------------------------------------------- index checks ---

// Index contents are preconditions; these checks run only when asked for
// (gdr_check_indices on host arrays, or every call once gdr_set_debug_checks
// is on).  -1: not decided yet (the environment decides on first use).
std::atomic<int> g_debug_checks{-1};

bool debug_checks_on() {
    int v = g_debug_checks.load(std::memory_order_relaxed);
    if (v < 0) {
        const char* e = std::getenv("GDR_DEBUG_CHECK_SLOTS");
        int want = (e != nullptr && std::strtol(e, nullptr, 10) != 0) ? 1 : 0;
        g_debug_checks.compare_exchange_strong(v, want);
        v = g_debug_checks.load(std::memory_order_relaxed);
    }
    return v > 0;
}

// Values of `idx` at the rows where `use` holds must be below `limit` and
// pairwise distinct.
template <typename Use>
int check_distinct_below(const char* fn, const char* what, int64_t rows, const uint32_t* idx,
                         int64_t limit, const char* limit_name, Use use) {
    std::vector<std::pair<uint32_t, int64_t>> seen;
    seen.reserve(static_cast<size_t>(rows));
    for (int64_t b = 0; b < rows; ++b) {
        if (!use(b)) continue;
        if (static_cast<int64_t>(idx[b]) >= limit)
            return fail(GDR_ERR_INVALID_ARG, "%s: %s %u of row %lld is not below the %lld %s", fn,
                        what, idx[b], static_cast<long long>(b), static_cast<long long>(limit),
                        limit_name);
        seen.emplace_back(idx[b], b);
    }
    std::sort(seen.begin(), seen.end());
    for (size_t i = 1; i < seen.size(); ++i)
        if (seen[i].first == seen[i - 1].first)
            return fail(GDR_ERR_INVALID_ARG, "%s: %s %u is used by rows %lld and %lld (two rows "
                        "on one %s race)", fn, what, seen[i].first,
                        static_cast<long long>(seen[i - 1].second),
                        static_cast<long long>(seen[i].second), what);
    return GDR_OK;
}

int check_indices_impl(const char* fn, int64_t rows, const uint32_t* off, int64_t total_tokens,
                       const uint32_t* slots, int64_t num_slots, const uint32_t* ring_idx,
                       int64_t ring_rows, int64_t ring_len, const uint32_t* accepted) {
    if (rows < 0) return fail(GDR_ERR_INVALID_ARG, "%s: negative row count", fn);
    if (off) {
        for (int64_t b = 0; b < rows; ++b)
            if (off[b + 1] < off[b])
                return fail(GDR_ERR_INVALID_ARG, "%s: row offsets decrease at row %lld (%u, then "
                            "%u)", fn, static_cast<long long>(b), off[b], off[b + 1]);
        if (static_cast<int64_t>(off[rows]) > total_tokens)
            return fail(GDR_ERR_INVALID_ARG, "%s: row offsets end at %u, past the %lld tokens", fn,
                        off[rows], static_cast<long long>(total_tokens));
    }
    auto active = [&](int64_t b) { return slots == nullptr || slots[b] != gdr::kPadSlot; };
    int rc;
    if (slots && (rc = check_distinct_below(fn, "slot", rows, slots, num_slots, "pool slots",
                                            active)))
        return rc;
    if (ring_idx && (accepted || off)) {
        auto uses_ring = [&](int64_t b) {
            if (!active(b)) return false;
            const int64_t n = accepted ? static_cast<int64_t>(accepted[b])
                                       : static_cast<int64_t>(off[b + 1]) - off[b];
            return n > 0 && n <= ring_len;
        };
        if ((rc = check_distinct_below(fn, "ring row", rows, ring_idx, ring_rows, "ring rows",
                                       uses_ring)))
            return rc;
    }
    return GDR_OK;
}

// Copies n index elements (u32 or i32 bits) of t to the host; synchronises
// the stream.  Debug checks only.
int fetch_indices(const char* fn, const char* name, const gdr_tensor* t, int64_t n,
                  hipStream_t stream, std::vector<uint32_t>& out) {
    out.assign(static_cast<size_t>(n), 0u);
    if (n == 0) return GDR_OK;
    hipError_t e = hipMemcpyAsync(out.data(), t->data, static_cast<size_t>(n) * sizeof(uint32_t),
                                  hipMemcpyDefault, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess)
        return fail(GDR_ERR_HIP, "%s: index check could not read %s: %s", fn, name,
                    hipGetErrorString(e));
    return GDR_OK;
}

// The checks of one call, on its device index vectors (nullptr: absent).
struct IndexCheck {
    const gdr_tensor* offsets = nullptr;
    int64_t total_tokens = 0;
    const gdr_tensor* slots = nullptr;
    int64_t num_slots = 0;
    const gdr_tensor* ring_idx = nullptr;
    int64_t ring_rows = 0, ring_len = 0;
    const gdr_tensor* accepted = nullptr;
};

int run_debug_check(const char* fn, int64_t rows, const IndexCheck& c, void* stream) {
    if (!debug_checks_on()) return GDR_OK;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    std::vector<uint32_t> off, sl, ring, acc;
    int rc;
    if ((c.offsets && (rc = fetch_indices(fn, "row offsets", c.offsets, rows + 1, s, off))) ||
        (c.slots && (rc = fetch_indices(fn, "slots", c.slots, rows, s, sl))) ||
        (c.ring_idx && (rc = fetch_indices(fn, "ring rows", c.ring_idx, rows, s, ring))) ||
        (c.accepted && (rc = fetch_indices(fn, "accepted counts", c.accepted, rows, s, acc))))
        return rc;
    return check_indices_impl(fn, rows, c.offsets ? off.data() : nullptr, c.total_tokens,
                              c.slots ? sl.data() : nullptr, c.num_slots,
                              c.ring_idx ? ring.data() : nullptr, c.ring_rows, c.ring_len,
                              c.accepted ? acc.data() : nullptr);
}

float resolve_scale(float scale, int64_t K) {
    if (!(scale > 0.0f)) return 1.0f / std::sqrt(static_cast<float>(K));
    return scale;
}

// Launch shape, by entry and row length: about one token per row -> decode
// tiles (one token per stage, high occupancy); short windows -> wider stages;
// the fused update on short rows (snapshot stores dominate) -> 16-byte state
// accesses; long rows (>= 16 tokens per row on average) -> narrow tiles, so
// the token-serial chain is spread over more waves.  The reduction order does
// not depend on this choice.
enum class Entry { Packed, Fused, Fold };

// Longest rows first for ragged multi-token batches small enough for every
// workgroup to rank the rows itself: for the short-row shapes (row groups in
// the high lane bits: verify windows) when the grid is larger than what one
// pass of the chip holds at once (256 compute units, about 4 workgroups
// each); for the long-row shapes always, because their rows share compute
// units with one another and the longest should start first.
int32_t order_rows(const gdr::LaunchShape& s, const gdr::RecParams& p) {
    const int64_t grid = int64_t{p.rows} * p.nk * p.parts;
    return p.offsets != nullptr && p.rows >= 2 && p.rows <= gdr::kOrderMaxRows &&
           s.chunk > 1 && (s.kg_low || grid > 4 * 256);
}

gdr::LaunchShape pick_shape(Entry e, int64_t K, int64_t V, int64_t G, int64_t total_tokens,
                            int64_t rows, int64_t nv) {
    gdr::LaunchShape s{};
    s.K = static_cast<int>(K);
    s.V = static_cast<int>(V);
    const bool long_rows = rows > 0 && total_tokens >= 16 * rows;
    const bool decode = rows > 0 && 2 * total_tokens <= 3 * rows;  // ~1 token per row
    if (K == 128 && K != V && e == Entry::Fused && !long_rows) {
        s.cpl = gdr::kFusedCpl;  // as the K == V == 128 fused profile
        s.chunk = gdr::kFusedChunk;
        s.kg_low = gdr::kFusedKgLow;
    } else if (K == 256 || K != V) {  // one short and one long-row shape per pair
        if (e == Entry::Fold || !long_rows) {
            s.cpl = K == 256 ? 2 : (K == 64 ? 8 : 4);
            s.chunk = e == Entry::Fold ? 1 : 8;
        } else {
            s.cpl = K == 64 ? 2 : 1;
            s.chunk = K == 256 ? 8 : 16;
            s.kg_low = true;
        }
    } else if (K == 128) {
        if (e == Entry::Fold) {
            s.cpl = gdr::kFoldCpl;
            s.chunk = 1;
        } else if (long_rows) {
            s.cpl = gdr::kLongCpl;
            s.chunk = gdr::kLongChunk;
            s.kg_low = gdr::kLongKgLow;
        } else if (e == Entry::Fused && !decode) {
            s.cpl = gdr::kFusedCpl;
            s.chunk = gdr::kFusedChunk;
            s.kg_low = gdr::kFusedKgLow;
        } else if (decode) {
            // A batch whose decode shape would give 256 waves or fewer (4 rows
            // at 32 value heads) is latency-bound: narrower tiles spread it
            // over 4x the waves.
            const bool tiny = rows * nv * (V / (gdr::kLanesPerRow * gdr::kDecodeCpl)) <= 256;
            s.cpl = tiny ? gdr::kTinyCpl : gdr::kDecodeCpl;
            s.chunk = gdr::kDecodeChunk;
            s.kg_low = gdr::kDecodeKgLow;
        } else {
            s.cpl = gdr::kShortCpl;
            s.chunk = gdr::kShortChunk;
            s.kg_low = gdr::kShortKgLow;
        }
    } else if (long_rows && e != Entry::Fold) {
        s.cpl = 2;
        s.chunk = 16;
        s.kg_low = true;
    } else {
        s.cpl = K == 64 ? 8 : (K == 32 ? 4 : 2);
        s.chunk = 8;
    }
    const int64_t tiles = V / (gdr::kLanesPerRow * s.cpl);
    const int64_t units = G * tiles;
    s.wpg = units % 4 == 0 ? 4 : (units % 2 == 0 ? 2 : 1);
    return s;
}

int hip_status(const char* fn, hipError_t e) {
    if (e != hipSuccess)
        return fail(GDR_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    g_last_error.clear();
    return GDR_OK;
}

const uint32_t* as_u32(const gdr_tensor* t) {
    return present(t) ? static_cast<const uint32_t*>(t->data) : nullptr;
}

// Shared by the forward and the verify entry points.
int packed_walk(const char* fn, int32_t nv, int32_t nk, const gdr_tensor* out,
                const gdr_tensor* state, const gdr_tensor* slot_idx, const gdr_tensor* qkv,
                const gdr_tensor* decay, const gdr_tensor* beta, const gdr_tensor* offsets,
                const gdr_tensor* ring, const gdr_tensor* ring_slot_idx, float scale,
                uint32_t flags, void* stream) {
    if (nk < 1 || nv < nk || nv % nk != 0)
        return fail(GDR_ERR_INVALID_ARG, "%s: num_value_heads (%d) must be a positive multiple "
                    "of num_key_heads (%d)", fn, nv, nk);
    if (flags & ~GDR_FLAG_L2NORM_QK)
        return fail(GDR_ERR_INVALID_ARG, "%s: unknown flags 0x%x", fn, flags);
    int rc;
    const int64_t st_shape[4] = {-1, nv, -1, -1};
    if ((rc = check_state(fn, "recurrent_state", state, 4, st_shape))) return rc;
    const int64_t K = state->shape[2], V = state->shape[3];
    if (missing(slot_idx)) return fail(GDR_ERR_INVALID_ARG, "%s: slot_idx is null", fn);
    const int64_t B = slot_idx->shape[0];
    if ((rc = check_index_vec(fn, "slot_idx", slot_idx, B))) return rc;
    if ((rc = check_index_vec(fn, "input_row_offsets", offsets, B + 1))) return rc;
    const int64_t conv = 2 * nk * K + nv * V;
    const int64_t qkv_shape[2] = {-1, conv};
    if ((rc = check_tensor(fn, "qkv_conv_output", qkv, 2, qkv_shape, true, true, false)))
        return rc;
    const int32_t work = qkv->dtype;
    if ((rc = check_layout(fn, "qkv_conv_output", qkv, vec_mult(work)))) return rc;
    const int64_t T = qkv->shape[0];
    const int64_t gate_shape[2] = {T, nv};
    if ((rc = check_tensor(fn, "decay_per_token", decay, 2, gate_shape, true, true, false)) ||
        (rc = check_work_dtype(fn, "decay_per_token", decay, work)))
        return rc;
    if ((rc = check_tensor(fn, "beta_per_token", beta, 2, gate_shape, true, true, false)) ||
        (rc = check_work_dtype(fn, "beta_per_token", beta, work)))
        return rc;
    const int64_t out_shape[2] = {T, nv * V};
    if ((rc = check_tensor(fn, "recurrence_output", out, 2, out_shape, true, true, false)) ||
        (rc = check_work_dtype(fn, "recurrence_output", out, work)))
        return rc;
    if ((rc = check_layout(fn, "recurrence_output", out, vec_mult(work)))) return rc;
    const int64_t G = nv / nk;

    gdr::RecParams p{};
    if (ring) {
        if ((rc = check_tensor(fn, "ring", ring, 4, nullptr, true, true, false))) return rc;
        if (ring->shape[1] != nk)
            return fail(GDR_ERR_INVALID_ARG, "%s: ring dim 1 must be num_key_heads", fn);
        if (ring->shape[2] < 1)
            return fail(GDR_ERR_INVALID_ARG, "%s: ring length must be >= 1", fn);
        if (ring->shape[3] < gdr_ring_record_elements(static_cast<int32_t>(G),
                                                      static_cast<int32_t>(K),
                                                      static_cast<int32_t>(V)))
            return fail(GDR_ERR_INVALID_ARG, "%s: ring record stride %lld below %lld", fn,
                        static_cast<long long>(ring->shape[3]),
                        static_cast<long long>(gdr_ring_record_elements(
                            static_cast<int32_t>(G), static_cast<int32_t>(K),
                            static_cast<int32_t>(V))));
        if ((rc = check_layout(fn, "ring", ring, ring->dtype == GDR_DTYPE_BF16 ? 8 : 4)))
            return rc;
        if ((rc = check_index_vec(fn, "ring_slot_idx", ring_slot_idx, B))) return rc;
        p.ring = ring->data;
        p.ring_bf16 = ring->dtype == GDR_DTYPE_BF16 ? 1 : 0;
        p.ring_idx = as_u32(ring_slot_idx);
        p.ring_row = ring->stride[0];
        p.ring_head = ring->stride[1];
        p.ring_tok = ring->stride[2];
        p.ring_len = static_cast<int32_t>(ring->shape[2]);
    }
    if (B == 0) {
        g_last_error.clear();
        return GDR_OK;
    }
    if (B * nk > (int64_t{1} << 28))
        return fail(GDR_ERR_INVALID_ARG, "%s: batch too large", fn);

    const gdr::LaunchShape s = pick_shape(Entry::Packed, K, V, G, T, B, nv);
    const int64_t units = G * (V / (gdr::kLanesPerRow * s.cpl));
    p.rows = static_cast<int32_t>(B);
    p.nv = nv;
    p.nk = nk;
    p.G = static_cast<int32_t>(G);
    p.parts = static_cast<int32_t>(units / s.wpg);
    p.div_parts = gdr::make_fastdiv(static_cast<uint32_t>(p.parts));
    p.div_nk = gdr::make_fastdiv(static_cast<uint32_t>(p.nk));
    p.div_row = gdr::make_fastdiv(static_cast<uint32_t>(p.parts * p.nk));
    if (int64_t{p.rows} * p.nk * p.parts > INT32_MAX)
        return fail(GDR_ERR_INVALID_ARG, "%s: batch too large for one launch", fn);
    p.offsets = as_u32(offsets);
    const char* x = static_cast<const char*>(qkv->data);
    const int64_t es = work == GDR_DTYPE_BF16 ? 2 : 4;
    const int64_t ch = qkv->stride[1];
    p.q = x;
    p.k = x + nk * K * ch * es;
    p.v = x + 2 * nk * K * ch * es;
    p.q_tok = p.k_tok = p.v_tok = qkv->stride[0];
    p.q_head = p.k_head = K;
    p.v_head = V;
    p.gate = decay->data;
    p.g_tok = decay->stride[0];
    p.g_head = decay->stride[1];
    p.gate_is_log = 0;
    p.beta = beta->data;
    p.b_tok = beta->stride[0];
    p.b_head = beta->stride[1];
    p.out = out->data;
    p.o_tok = out->stride[0];
    p.o_head = V;
    p.slot_idx = as_u32(slot_idx);
    p.src = state->data;
    p.src_slot = state->stride[0];
    p.src_head = state->stride[1];
    p.src_by_slot = 1;
    p.dst = state->data;
    p.dst_slot = state->stride[0];
    p.dst_head = state->stride[1];
    p.dst_by_slot = 1;
    p.spt = 1;
    p.scale = resolve_scale(scale, K);
    p.l2norm = (flags & GDR_FLAG_L2NORM_QK) ? 1 : 0;
    p.order = order_rows(s, p);
    IndexCheck ic;
    ic.offsets = offsets;
    ic.total_tokens = T;
    ic.slots = slot_idx;
    ic.num_slots = state->shape[0];
    if (ring) {
        ic.ring_idx = ring_slot_idx;
        ic.ring_rows = ring->shape[0];
        ic.ring_len = ring->shape[2];
    }
    if ((rc = run_debug_check(fn, B, ic, stream))) return rc;
    const gdr::StateType st =
        state->dtype == GDR_DTYPE_BF16 ? gdr::StateType::BF16 : gdr::StateType::F32;
    return hip_status(fn, gdr::launch_recurrence(p, s, st, work == GDR_DTYPE_BF16,
                                                 static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int gdr_recurrence_fwd(int32_t num_value_heads, int32_t num_key_heads,
                       const gdr_tensor* recurrence_output, const gdr_tensor* recurrent_state,
                       const gdr_tensor* slot_idx, const gdr_tensor* qkv_conv_output,
                       const gdr_tensor* decay_per_token, const gdr_tensor* beta_per_token,
                       const gdr_tensor* input_row_offsets, float scale, uint32_t flags,
                       void* stream) {
    return packed_walk("gdr_recurrence_fwd", num_value_heads, num_key_heads, recurrence_output,
                       recurrent_state, slot_idx, qkv_conv_output, decay_per_token,
                       beta_per_token, input_row_offsets, nullptr, nullptr, scale, flags,
                       stream);
}

int gdr_recurrence_verify_ring(int32_t num_value_heads, int32_t num_key_heads,
                               const gdr_tensor* recurrence_output,
                               const gdr_tensor* recurrent_state, const gdr_tensor* slot_idx,
                               const gdr_tensor* qkv_conv_output,
                               const gdr_tensor* decay_per_token,
                               const gdr_tensor* beta_per_token,
                               const gdr_tensor* input_row_offsets, const gdr_tensor* ring,
                               const gdr_tensor* ring_slot_idx, float scale, uint32_t flags,
                               void* stream) {
    const char* fn = "gdr_recurrence_verify_ring";
    if (missing(ring)) return fail(GDR_ERR_INVALID_ARG, "%s: ring is null", fn);
    return packed_walk(fn, num_value_heads, num_key_heads, recurrence_output, recurrent_state,
                       slot_idx, qkv_conv_output, decay_per_token, beta_per_token,
                       input_row_offsets, ring, ring_slot_idx, scale, flags, stream);
}

int gdr_state_fold(int32_t num_value_heads, int32_t num_key_heads,
                   const gdr_tensor* recurrent_state, const gdr_tensor* slot_idx,
                   const gdr_tensor* ring, const gdr_tensor* ring_slot_idx,
                   const gdr_tensor* accepted, void* stream) {
    const char* fn = "gdr_state_fold";
    const int32_t nv = num_value_heads, nk = num_key_heads;
    if (nk < 1 || nv < nk || nv % nk != 0)
        return fail(GDR_ERR_INVALID_ARG, "%s: num_value_heads (%d) must be a positive multiple "
                    "of num_key_heads (%d)", fn, nv, nk);
    int rc;
    const int64_t st_shape[4] = {-1, nv, -1, -1};
    if ((rc = check_state(fn, "recurrent_state", recurrent_state, 4, st_shape))) return rc;
    const int64_t K = recurrent_state->shape[2], V = recurrent_state->shape[3];
    if (missing(slot_idx)) return fail(GDR_ERR_INVALID_ARG, "%s: slot_idx is null", fn);
    const int64_t B = slot_idx->shape[0];
    if ((rc = check_index_vec(fn, "slot_idx", slot_idx, B))) return rc;
    if ((rc = check_index_vec(fn, "ring_slot_idx", ring_slot_idx, B))) return rc;
    if ((rc = check_index_vec(fn, "accepted", accepted, B))) return rc;
    if ((rc = check_tensor(fn, "ring", ring, 4, nullptr, true, true, false))) return rc;
    const int64_t G = nv / nk;
    if (ring->shape[1] != nk)
        return fail(GDR_ERR_INVALID_ARG, "%s: ring dim 1 must be num_key_heads", fn);
    if (ring->shape[2] < 1) return fail(GDR_ERR_INVALID_ARG, "%s: ring length must be >= 1", fn);
    if (ring->shape[3] < gdr_ring_record_elements(static_cast<int32_t>(G),
                                                  static_cast<int32_t>(K),
                                                  static_cast<int32_t>(V)))
        return fail(GDR_ERR_INVALID_ARG, "%s: ring record stride too small", fn);
    if ((rc = check_layout(fn, "ring", ring, ring->dtype == GDR_DTYPE_BF16 ? 8 : 4))) return rc;
    if (B == 0) {
        g_last_error.clear();
        return GDR_OK;
    }
    gdr::LaunchShape s = pick_shape(Entry::Fold, K, V, G, B, B, nv);
    if (K == 128 && V == 128 && ring->dtype == GDR_DTYPE_BF16) {
        s.cpl = gdr::kFoldCplBf16Ring;  // 16-byte state accesses (measured faster with a bf16 ring)
        const int64_t units16 = G * (V / (gdr::kLanesPerRow * s.cpl));
        s.wpg = units16 % 4 == 0 ? 4 : (units16 % 2 == 0 ? 2 : 1);
    }
    const int64_t units = G * (V / (gdr::kLanesPerRow * s.cpl));
    gdr::FoldParams p{};
    p.rows = static_cast<int32_t>(B);
    p.nv = nv;
    p.nk = nk;
    p.G = static_cast<int32_t>(G);
    p.parts = static_cast<int32_t>(units / s.wpg);
    if (int64_t{p.rows} * p.nk * p.parts > INT32_MAX)
        return fail(GDR_ERR_INVALID_ARG, "%s: batch too large for one launch", fn);
    p.slot_idx = as_u32(slot_idx);
    p.state = recurrent_state->data;
    p.st_slot = recurrent_state->stride[0];
    p.st_head = recurrent_state->stride[1];
    p.ring = ring->data;
    p.ring_bf16 = ring->dtype == GDR_DTYPE_BF16 ? 1 : 0;
    p.ring_idx = as_u32(ring_slot_idx);
    p.ring_row = ring->stride[0];
    p.ring_head = ring->stride[1];
    p.ring_tok = ring->stride[2];
    p.ring_len = static_cast<int32_t>(ring->shape[2]);
    p.accepted = as_u32(accepted);
    IndexCheck ic;
    ic.slots = slot_idx;
    ic.num_slots = recurrent_state->shape[0];
    ic.ring_idx = ring_slot_idx;
    ic.ring_rows = ring->shape[0];
    ic.ring_len = ring->shape[2];
    ic.accepted = accepted;
    if ((rc = run_debug_check(fn, B, ic, stream))) return rc;
    const gdr::StateType st =
        recurrent_state->dtype == GDR_DTYPE_BF16 ? gdr::StateType::BF16 : gdr::StateType::F32;
    return hip_status(fn, gdr::launch_fold(p, s, st, static_cast<hipStream_t>(stream)));
}

int gdr_fused_recurrent_update(const gdr_tensor* q, const gdr_tensor* k, const gdr_tensor* v,
                               const gdr_tensor* g, const gdr_tensor* beta, float scale,
                               const gdr_tensor* initial_state, const gdr_tensor* final_state,
                               uint32_t flags, const gdr_tensor* cu_seqlens,
                               const gdr_tensor* state, const gdr_tensor* state_indices,
                               const gdr_tensor* intermediate_states, int32_t steps_per_token,
                               const gdr_tensor* o, void* stream) {
    const char* fn = "gdr_fused_recurrent_update";
    int rc;
    if (flags & ~GDR_FLAG_L2NORM_QK)
        return fail(GDR_ERR_INVALID_ARG, "%s: unknown flags 0x%x", fn, flags);
    if ((rc = check_tensor(fn, "q", q, 4, nullptr, true, true, false))) return rc;
    const int32_t work = q->dtype;
    const int64_t B = q->shape[0], T = q->shape[1], H = q->shape[2], K = q->shape[3];
    if ((rc = check_tensor(fn, "k", k, 4, q->shape, true, true, false)) ||
        (rc = check_work_dtype(fn, "k", k, work)))
        return rc;
    if ((rc = check_tensor(fn, "v", v, 4, nullptr, true, true, false)) ||
        (rc = check_work_dtype(fn, "v", v, work)))
        return rc;
    const int64_t HV = v->shape[2], V = v->shape[3];
    if (v->shape[0] != B || v->shape[1] != T)
        return fail(GDR_ERR_INVALID_ARG, "%s: v must be [B, T, HV, V] like q", fn);
    if (H < 1 || HV < H || HV % H != 0)
        return fail(GDR_ERR_INVALID_ARG, "%s: HV must be a positive multiple of H", fn);
    if (!dims_built(K, V, true))
        return fail(GDR_ERR_UNSUPPORTED, "%s: head dims K=%lld V=%lld not built (%s)", fn,
                    static_cast<long long>(K), static_cast<long long>(V), kDimsBuilt);
    if ((rc = check_layout(fn, "q", q, vec_mult(work))) ||
        (rc = check_layout(fn, "k", k, vec_mult(work))) ||
        (rc = check_layout(fn, "v", v, vec_mult(work))))
        return rc;
    const int64_t gshape[3] = {B, T, HV};
    if (present(g) && ((rc = check_tensor(fn, "g", g, 3, gshape, true, true, false)) ||
                       (rc = check_work_dtype(fn, "g", g, work))))
        return rc;
    const bool beta_cols = present(beta) && beta->ndim == 4;
    if (beta_cols) {  // one beta per value column: [B, T, HV, V]
        if ((rc = check_tensor(fn, "beta", beta, 4, v->shape, true, true, false)) ||
            (rc = check_work_dtype(fn, "beta", beta, work)))
            return rc;
        if ((rc = check_layout(fn, "beta", beta, vec_mult(work)))) return rc;
    } else if (present(beta)) {
        if ((rc = check_tensor(fn, "beta", beta, 3, gshape, true, true, false)) ||
            (rc = check_work_dtype(fn, "beta", beta, work)))
            return rc;
    }
    const int64_t oshape[4] = {B, T, HV, V};
    if ((rc = check_tensor(fn, "o", o, 4, oshape, true, true, false)) ||
        (rc = check_work_dtype(fn, "o", o, work)))
        return rc;
    if ((rc = check_layout(fn, "o", o, vec_mult(work)))) return rc;

    int64_t N = B;
    if (present(cu_seqlens)) {
        if (B != 1) return fail(GDR_ERR_INVALID_ARG, "%s: cu_seqlens needs B == 1", fn);
        N = cu_seqlens->shape[0] - 1;
        if (N < 0) return fail(GDR_ERR_INVALID_ARG, "%s: cu_seqlens is empty", fn);
        if ((rc = check_index_vec(fn, "cu_seqlens", cu_seqlens, N + 1))) return rc;
    }
    if (steps_per_token < 1)
        return fail(GDR_ERR_INVALID_ARG, "%s: steps_per_token must be >= 1", fn);

    gdr::RecParams p{};
    int32_t st_dtype = -1;
    if (present(state)) {
        const int64_t sshape[4] = {-1, HV, K, V};
        if ((rc = check_state(fn, "state", state, 4, sshape, true))) return rc;
        st_dtype = state->dtype;
        p.src = p.dst = state->data;
        p.src_slot = p.dst_slot = state->stride[0];
        p.src_head = p.dst_head = state->stride[1];
        p.src_by_slot = p.dst_by_slot = 1;
        if (present(state_indices)) {
            if ((rc = check_index_vec(fn, "state_indices", state_indices, N))) return rc;
            p.slot_idx = as_u32(state_indices);
        } else if (N > state->shape[0]) {
            return fail(GDR_ERR_INVALID_ARG, "%s: state has fewer slots than sequences", fn);
        }
        if (present(intermediate_states)) {
            const int64_t ishape[5] = {state->shape[0], -1, HV, K, V};
            if ((rc = check_state(fn, "intermediate_states", intermediate_states, 5, ishape, true)))
                return rc;
            if (intermediate_states->dtype != st_dtype)
                return fail(GDR_ERR_UNSUPPORTED, "%s: intermediate_states must match the state "
                            "dtype", fn);
            p.snap = intermediate_states->data;
            p.snap_slot = intermediate_states->stride[0];
            p.snap_tok = intermediate_states->stride[1];
            p.snap_head = intermediate_states->stride[2];
            p.snap_count = static_cast<int32_t>(intermediate_states->shape[1]);
        }
    } else {
        if (present(intermediate_states))
            return fail(GDR_ERR_INVALID_ARG, "%s: intermediate_states needs state", fn);
        const int64_t dshape[4] = {N, HV, K, V};
        if (present(initial_state)) {
            if ((rc = check_state(fn, "initial_state", initial_state, 4, dshape, true))) return rc;
            st_dtype = initial_state->dtype;
            p.src = initial_state->data;
            p.src_slot = initial_state->stride[0];
            p.src_head = initial_state->stride[1];
        }
        if (present(final_state)) {
            if ((rc = check_state(fn, "final_state", final_state, 4, dshape, true))) return rc;
            if (st_dtype >= 0 && final_state->dtype != st_dtype)
                return fail(GDR_ERR_UNSUPPORTED, "%s: initial and final state dtypes differ", fn);
            st_dtype = final_state->dtype;
            p.dst = final_state->data;
            p.dst_slot = final_state->stride[0];
            p.dst_head = final_state->stride[1];
        }
    }
    if (N == 0 || (T == 0 && !present(cu_seqlens))) {
        g_last_error.clear();
        return GDR_OK;
    }
    if (N * H > (int64_t{1} << 28)) return fail(GDR_ERR_INVALID_ARG, "%s: batch too large", fn);

    const int64_t G = HV / H;
    const gdr::LaunchShape s = pick_shape(Entry::Fused, K, V, G, B * T, N, HV);
    const int64_t units = G * (V / (gdr::kLanesPerRow * s.cpl));
    p.rows = static_cast<int32_t>(N);
    p.nv = static_cast<int32_t>(HV);
    p.nk = static_cast<int32_t>(H);
    p.G = static_cast<int32_t>(G);
    p.parts = static_cast<int32_t>(units / s.wpg);
    p.div_parts = gdr::make_fastdiv(static_cast<uint32_t>(p.parts));
    p.div_nk = gdr::make_fastdiv(static_cast<uint32_t>(p.nk));
    p.div_row = gdr::make_fastdiv(static_cast<uint32_t>(p.parts * p.nk));
    if (int64_t{p.rows} * p.nk * p.parts > INT32_MAX)
        return fail(GDR_ERR_INVALID_ARG, "%s: batch too large for one launch", fn);
    p.dense_len = static_cast<int32_t>(T);
    p.offsets = as_u32(cu_seqlens);
    p.q = q->data;
    p.q_seq = q->stride[0]; p.q_tok = q->stride[1]; p.q_head = q->stride[2];
    p.k = k->data;
    p.k_seq = k->stride[0]; p.k_tok = k->stride[1]; p.k_head = k->stride[2];
    p.v = v->data;
    p.v_seq = v->stride[0]; p.v_tok = v->stride[1]; p.v_head = v->stride[2];
    if (present(g)) {
        p.gate = g->data;
        p.g_seq = g->stride[0]; p.g_tok = g->stride[1]; p.g_head = g->stride[2];
        p.gate_is_log = 1;
    }
    if (present(beta)) {
        p.beta = beta->data;
        p.b_seq = beta->stride[0]; p.b_tok = beta->stride[1]; p.b_head = beta->stride[2];
        p.beta_cols = beta_cols ? 1 : 0;
    }
    p.out = o->data;
    p.o_seq = o->stride[0]; p.o_tok = o->stride[1]; p.o_head = o->stride[2];
    p.spt = steps_per_token;
    p.scale = resolve_scale(scale, K);
    p.l2norm = (flags & GDR_FLAG_L2NORM_QK) ? 1 : 0;
    p.order = order_rows(s, p);
    IndexCheck ic;
    if (present(cu_seqlens)) {
        ic.offsets = cu_seqlens;
        ic.total_tokens = T;
    }
    if (present(state) && present(state_indices)) {
        ic.slots = state_indices;
        ic.num_slots = state->shape[0];
    }
    if ((rc = run_debug_check(fn, N, ic, stream))) return rc;
    const gdr::StateType st =
        st_dtype == GDR_DTYPE_BF16 ? gdr::StateType::BF16 : gdr::StateType::F32;
    return hip_status(fn, gdr::launch_recurrence(p, s, st, work == GDR_DTYPE_BF16,
                                                 static_cast<hipStream_t>(stream)));
}

int gdr_snapshot_rollback(const gdr_tensor* state, const gdr_tensor* state_indices,
                          const gdr_tensor* intermediate_states, const gdr_tensor* accepted,
                          void* stream) {
    const char* fn = "gdr_snapshot_rollback";
    int rc;
    if ((rc = check_state(fn, "state", state, 4, nullptr, true))) return rc;
    const int64_t S = state->shape[0], HV = state->shape[1], K = state->shape[2],
                  V = state->shape[3];
    const int64_t ishape[5] = {S, -1, HV, K, V};
    if ((rc = check_state(fn, "intermediate_states", intermediate_states, 5, ishape, true)))
        return rc;
    if (intermediate_states->dtype != state->dtype)
        return fail(GDR_ERR_UNSUPPORTED, "%s: intermediate_states must match the state dtype", fn);
    if (missing(state_indices)) return fail(GDR_ERR_INVALID_ARG, "%s: state_indices is null", fn);
    const int64_t N = state_indices->shape[0];
    if ((rc = check_index_vec(fn, "state_indices", state_indices, N))) return rc;
    if ((rc = check_index_vec(fn, "accepted", accepted, N))) return rc;
    if (N == 0 || HV == 0 || intermediate_states->shape[1] == 0) {
        g_last_error.clear();
        return GDR_OK;
    }
    const int64_t es = state->dtype == GDR_DTYPE_BF16 ? 2 : 4;
    const int64_t block16 = K * V * es / 16;
    const int64_t per_wg = int64_t{gdr::kRollbackThreads} * gdr::kRollbackPerThread;
    gdr::RollbackParams p{};
    p.rows = static_cast<int32_t>(N);
    p.HV = static_cast<int32_t>(HV);
    p.chunks = static_cast<int32_t>((block16 + per_wg - 1) / per_wg);
    if (N * HV * p.chunks > (int64_t{1} << 31) - 1)
        return fail(GDR_ERR_INVALID_ARG, "%s: batch too large", fn);
    p.idx = static_cast<const int32_t*>(state_indices->data);
    p.accepted = static_cast<const int32_t*>(accepted->data);
    p.state = state->data;
    p.st_slot = state->stride[0] * es;
    p.st_head = state->stride[1] * es;
    p.inter = intermediate_states->data;
    p.in_slot = intermediate_states->stride[0] * es;
    p.in_tok = intermediate_states->stride[1] * es;
    p.in_head = intermediate_states->stride[2] * es;
    p.int_tokens = static_cast<int32_t>(intermediate_states->shape[1]);
    p.block16 = block16;
    IndexCheck ic;
    ic.slots = state_indices;
    ic.num_slots = S;
    if ((rc = run_debug_check(fn, N, ic, stream))) return rc;
    return hip_status(fn, gdr::launch_rollback(p, static_cast<hipStream_t>(stream)));
}

int gdr_causal_conv1d(const gdr_tensor* out, const gdr_tensor* x, const gdr_tensor* weight,
                      const gdr_tensor* bias, const gdr_tensor* conv_state,
                      const gdr_tensor* slot_idx, const gdr_tensor* input_row_offsets,
                      uint32_t flags, void* stream) {
    const char* fn = "gdr_causal_conv1d";
    int rc;
    if (flags & ~GDR_FLAG_CONV_SILU)
        return fail(GDR_ERR_INVALID_ARG, "%s: unknown flags 0x%x", fn, flags);
    if ((rc = check_tensor(fn, "x", x, 2, nullptr, true, true, false))) return rc;
    const int32_t work = x->dtype;
    const int64_t T = x->shape[0], C = x->shape[1];
    if (C % 4 != 0) return fail(GDR_ERR_UNSUPPORTED, "%s: channels must be a multiple of 4", fn);
    if ((rc = check_layout(fn, "x", x, 4))) return rc;
    if ((rc = check_tensor(fn, "out", out, 2, x->shape, true, true, false)) ||
        (rc = check_work_dtype(fn, "out", out, work)) || (rc = check_layout(fn, "out", out, 4)))
        return rc;
    if (out->data == x->data && !empty(x))
        return fail(GDR_ERR_INVALID_ARG, "%s: out must not alias x", fn);
    const int64_t wshape[2] = {C, -1};
    if ((rc = check_tensor(fn, "weight", weight, 2, wshape, true, false, false))) return rc;
    const int64_t W = weight->shape[1];
    if (W < 2 || W > 4)
        return fail(GDR_ERR_UNSUPPORTED, "%s: kernel width %lld not built (2, 3, 4)", fn,
                    static_cast<long long>(W));
    if (weight->stride[1] != 1 && !empty(weight))
        return fail(GDR_ERR_UNSUPPORTED, "%s: weight needs unit stride over the taps", fn);
    const int64_t cshape[1] = {C};
    if (present(bias) && ((rc = check_tensor(fn, "bias", bias, 1, cshape, true, false, false))))
        return rc;
    if (present(bias) && C > 1 && bias->stride[0] != 1)
        return fail(GDR_ERR_UNSUPPORTED, "%s: bias must be contiguous", fn);
    if ((rc = check_tensor(fn, "input_row_offsets", input_row_offsets, 1, nullptr, false, false,
                           true)))
        return rc;
    const int64_t B = input_row_offsets->shape[0] - 1;
    if (B < 0) return fail(GDR_ERR_INVALID_ARG, "%s: input_row_offsets is empty", fn);
    if ((rc = check_index_vec(fn, "input_row_offsets", input_row_offsets, B + 1))) return rc;
    if (present(slot_idx) && (rc = check_index_vec(fn, "slot_idx", slot_idx, B))) return rc;
    gdr::ConvParams p{};
    if (present(conv_state)) {
        const int64_t sshape[3] = {-1, W - 1, C};
        if ((rc = check_tensor(fn, "conv_state", conv_state, 3, sshape, true, true, false)) ||
            (rc = check_work_dtype(fn, "conv_state", conv_state, work)) ||
            (rc = check_layout(fn, "conv_state", conv_state, 4)))
            return rc;
        if (!present(slot_idx) && conv_state->shape[0] < B)
            return fail(GDR_ERR_INVALID_ARG, "%s: conv_state has fewer slots than rows", fn);
        p.state = conv_state->data;
        p.st_slot = conv_state->stride[0];
        p.st_tok = conv_state->stride[1];
    }
    if (B == 0 || T == 0 || C == 0) {
        g_last_error.clear();
        return GDR_OK;
    }
    if (T > (int64_t{1} << 31) - 1 || B > (int64_t{1} << 20))
        return fail(GDR_ERR_INVALID_ARG, "%s: too many tokens or rows", fn);
    p.B = static_cast<int32_t>(B);
    p.C = static_cast<int32_t>(C);
    p.T = static_cast<int32_t>(T);
    p.W = static_cast<int32_t>(W);
    p.silu = (flags & GDR_FLAG_CONV_SILU) ? 1 : 0;
    p.offsets = as_u32(input_row_offsets);
    p.slot_idx = as_u32(slot_idx);
    p.x = x->data;
    p.x_tok = x->stride[0];
    p.out = out->data;
    p.o_tok = out->stride[0];
    p.weight = static_cast<const float*>(weight->data);
    p.w_chan = weight->stride[0];
    p.bias = present(bias) ? static_cast<const float*>(bias->data) : nullptr;
    IndexCheck ic;
    ic.offsets = input_row_offsets;
    ic.total_tokens = T;
    if (present(conv_state) && present(slot_idx)) {
        ic.slots = slot_idx;
        ic.num_slots = conv_state->shape[0];
    }
    if ((rc = run_debug_check(fn, B, ic, stream))) return rc;
    return hip_status(fn, gdr::launch_conv(p, work == GDR_DTYPE_BF16,
                                           static_cast<hipStream_t>(stream)));
}

int gdr_fwd_output_shape(const gdr_tensor* qkv_conv_output, const gdr_tensor* recurrent_state,
                         int64_t out_shape[2]) {
    const char* fn = "gdr_fwd_output_shape";
    if (!qkv_conv_output || !recurrent_state || !out_shape)
        return fail(GDR_ERR_INVALID_ARG, "%s: null argument", fn);
    if (qkv_conv_output->ndim != 2 || recurrent_state->ndim != 4)
        return fail(GDR_ERR_INVALID_ARG, "%s: expected qkv rank 2 and state rank 4", fn);
    out_shape[0] = qkv_conv_output->shape[0];
    out_shape[1] = recurrent_state->shape[1] * recurrent_state->shape[3];
    g_last_error.clear();
    return GDR_OK;
}

int64_t gdr_ring_record_elements(int32_t group, int32_t key_head_dim, int32_t value_head_dim) {
    if (group < 1 || key_head_dim < 1 || value_head_dim < 1) return -1;
    return static_cast<int64_t>(key_head_dim) +
           static_cast<int64_t>(group) * (static_cast<int64_t>(value_head_dim) + 1);
}

int gdr_check_indices(int64_t rows, const uint32_t* row_offsets, int64_t total_tokens,
                      const uint32_t* slots, int64_t num_slots, const uint32_t* ring_idx,
                      int64_t ring_rows, int64_t ring_len, const uint32_t* accepted) {
    const int rc = check_indices_impl("gdr_check_indices", rows, row_offsets, total_tokens, slots,
                                      num_slots, ring_idx, ring_rows, ring_len, accepted);
    if (rc == GDR_OK) g_last_error.clear();
    return rc;
}

int gdr_set_debug_checks(int enable) {
    const int before = debug_checks_on() ? 1 : 0;
    g_debug_checks.store(enable ? 1 : 0, std::memory_order_relaxed);
    return before;
}

const char* gdr_last_error_message(void) { return g_last_error.c_str(); }

const char* gdr_version(void) { return "gdr 0.1.0 gfx950"; }

}  // extern "C"
