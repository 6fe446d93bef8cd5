/*
 * Plain CPU oracle for the gated delta rule recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously correct
 * reference that the tests, the smoke check and the benchmark's CPU-baseline
 * leg compare the HIP library against.  Nothing in the product path may link,
 * load or call it, and it shares no source, header, table or helper with the
 * HIP library.
 *
 * Sources (the four documentation pages the method is described on):
 *   [fwd]    "gated_delta_recurrence_fwd_gpu" (Mojo kernel API page):
 *            summary paragraph and Args (slot-indexed ragged forward).
 *   [verify] "gated_delta_recurrence_verify_ring_gpu" (Mojo kernel API page):
 *            summary paragraphs, Parameters (ring_dtype) and Args (ring).
 *   [shape]  "gated_delta_recurrence_fwd_shape" (Mojo graph-op page).
 *   [gdp]    "core.ssm.ops.gdp.fused_recurrent" (Megatron Core API page):
 *            module summary, fused_recurrent_gated_delta_rule_update
 *            parameters.
 * The Pass-1 causal Conv1d that produces the fwd page's qkv_conv_output is
 * only named there; oracle_causal_conv1d states the reading it implements.
 * Parity unpinned against the pages for that reading (nothing on them fixes
 * the step); its arithmetic is pinned by exact delays, numpy's convolve and
 * split-call continuity.
 *
 * The recurrence (per sequence and value head, a K x V state S carried token
 * by token; the pages call it the gated delta rule and describe the state as
 * "[K, V]" with a per-token decay factor and beta gate):
 *     S  <- a_t * S                      (decay)
 *     r  =  S^T k_t                      (retrieval, one value per V column)
 *     u  =  beta_t * (v_t - r)           (delta correction)
 *     S  <- S + k_t u^T                  (rank-1 write)
 *     o_t = scale * S^T q_t              (read-out, after the write)
 * with q_t and k_t optionally L2-normalised first, and scale defaulting to
 * 1/sqrt(K).  Everything is written in this order, in float32 (the work dtype
 * the fwd page fixes), one scalar operation at a time, with contraction off
 * (built with -ffp-contract=off) so that no fused multiply-add appears.
 *
 * Readings of points the pages leave open:
 *   - L2 norm: x * (1 / sqrt(sum x^2 + eps)) with eps = 1e-6.
 *   - GQA: value head hv reads key head hv / (nv / nk).  Parity unpinned
 *     against the pages (a convention; pinned only by replicated heads).
 *   - bf16 state stores round to nearest even, once per store; loads widen.
 *   - Slot index 0xFFFFFFFF (-1 as int32) is a padding request in every
 *     entry: zero output, no state, ring or snapshot access.
 *   - Ring record (verify page: each token's record holds what the fold uses):
 *       [ k_hat (K) | u of value head h*G+m, m < G (G*V) | a of those heads (G) ]
 *     so the fold needs no norm, exp or reduction.  Parity unpinned for the
 *     layout (the page fixes only its size's dependence on nv / nk).
 *   - Fold count: per-row accepted[b]; 0 or > RING_LEN leaves the state alone.
 */
#include <math.h>
#include <pthread.h>
#include <stdatomic.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_L2NORM_EPS 1e-6f
#define ORACLE_PAD_SLOT 0xFFFFFFFFu

/* ---------------------------------------------------------------- bf16 --- */

/* Round a float32 to bfloat16, nearest-even on the dropped 16 bits.  NaN stays
 * a (quiet) NaN. */
static uint16_t oracle_bf16_round(float f)
{
    uint32_t x;
    memcpy(&x, &f, sizeof x);
    if ((x & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((x >> 16) | 0x0040u);
    uint32_t keep_lsb = (x >> 16) & 1u;
    x += 0x7fffu + keep_lsb;
    return (uint16_t)(x >> 16);
}

static float oracle_bf16_widen(uint16_t h)
{
    uint32_t x = (uint32_t)h << 16;
    float f;
    memcpy(&f, &x, sizeof f);
    return f;
}

/* Exposed so the tests can pin the rounding against a library conversion. */
void oracle_bf16_round_array(const float* in, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_round(in[i]);
}

/* A K*V block of state in either float32 or bfloat16 storage. */
static void oracle_load_block(const void* base, int bf16, int64_t offset, int64_t n, float* dst)
{
    if (bf16) {
        const uint16_t* p = (const uint16_t*)base + offset;
        for (int64_t i = 0; i < n; ++i)
            dst[i] = oracle_bf16_widen(p[i]);
    } else {
        const float* p = (const float*)base + offset;
        for (int64_t i = 0; i < n; ++i)
            dst[i] = p[i];
    }
}

static void oracle_store_block(void* base, int bf16, int64_t offset, int64_t n, const float* src)
{
    if (bf16) {
        uint16_t* p = (uint16_t*)base + offset;
        for (int64_t i = 0; i < n; ++i)
            p[i] = oracle_bf16_round(src[i]);
    } else {
        float* p = (float*)base + offset;
        for (int64_t i = 0; i < n; ++i)
            p[i] = src[i];
    }
}

/* One ring element, stored as float32 or rounded to bfloat16 ([verify]
 * Parameters, ring_dtype). */
static void oracle_ring_put(void* ring, int ring_bf16, int64_t i, float v)
{
    if (ring_bf16)
        ((uint16_t*)ring)[i] = oracle_bf16_round(v);
    else
        ((float*)ring)[i] = v;
}

static float oracle_ring_get(const void* ring, int ring_bf16, int64_t i)
{
    return ring_bf16 ? oracle_bf16_widen(((const uint16_t*)ring)[i]) : ((const float*)ring)[i];
}

/* ------------------------------------------------------------ one step --- */

/* x_hat = x / sqrt(sum x^2 + eps), written as a multiply by the reciprocal
 * root ([fwd] summary: the norm is a scalar factor). */
static void oracle_l2norm(int n, const float* x, float* out)
{
    float sq = 0.0f;
    for (int i = 0; i < n; ++i)
        sq = sq + x[i] * x[i];
    float rho = 1.0f / sqrtf(sq + ORACLE_L2NORM_EPS);
    for (int i = 0; i < n; ++i)
        out[i] = x[i] * rho;
}

/*
 * One recurrence step on S (K rows, V columns, row-major, V fastest).
 *   khat, qhat: the (already normalised, if enabled) key and query, length K.
 *   v:          the value, length V.
 *   a:          decay factor.
 *   beta:       beta gate; a single value, or V values when beta_per_v.
 *   o:          V outputs (scale * S^T qhat after the write), or NULL.
 *   u_out:      receives u (V values) when not NULL.
 */
static void oracle_step(int K, int V, float* S, const float* khat, const float* qhat,
                        const float* v, float a, const float* beta, int beta_per_v,
                        float scale, float* o, float* u_out)
{
    float* u = (float*)malloc(sizeof(float) * (size_t)V);

    for (int i = 0; i < K; ++i)
        for (int j = 0; j < V; ++j)
            S[i * V + j] = a * S[i * V + j];

    for (int j = 0; j < V; ++j) {
        float r = 0.0f;
        for (int i = 0; i < K; ++i)
            r = r + S[i * V + j] * khat[i];
        float b = beta_per_v ? beta[j] : beta[0];
        u[j] = b * (v[j] - r);
    }

    for (int i = 0; i < K; ++i)
        for (int j = 0; j < V; ++j)
            S[i * V + j] = S[i * V + j] + khat[i] * u[j];

    if (o) {
        for (int j = 0; j < V; ++j) {
            float acc = 0.0f;
            for (int i = 0; i < K; ++i)
                acc = acc + S[i * V + j] * qhat[i];
            o[j] = scale * acc;
        }
    }
    if (u_out)
        for (int j = 0; j < V; ++j)
            u_out[j] = u[j];
    free(u);
}

/* Fetch and optionally normalise q_t, k_t of key head h from the packed conv
 * output row ([fwd] Args, qkv_conv_output: the queries of all key heads come
 * first, then the keys, then the values, so q of key head h starts at channel
 * h*K, k at nk*K + h*K and v of value head hv at 2*nk*K + hv*V). */
static void oracle_packed_qk(const float* row, int nk, int K, int h, int l2norm,
                             float* qhat, float* khat)
{
    const float* q = row + (int64_t)h * K;
    const float* k = row + (int64_t)nk * K + (int64_t)h * K;
    if (l2norm) {
        oracle_l2norm(K, q, qhat);
        oracle_l2norm(K, k, khat);
    } else {
        for (int i = 0; i < K; ++i) {
            qhat[i] = q[i];
            khat[i] = k[i];
        }
    }
}

/* ------------------------------------------------- work-item farm ------ */

/*
 * Every (sequence, value head) pair is an independent recurrence: it reads and
 * writes only its own state block, output columns and ring elements (slots
 * are distinct by precondition).  The walks below are therefore written as
 * one function per work item, and oracle_farm runs items 0..items-1 either in
 * order on the calling thread (threads <= 1) or spread over a few threads
 * that take the next item from a shared counter.  Either way each item runs
 * the same single-threaded code, so the results are identical.
 */
typedef int (*oracle_item_fn)(const void* args, int64_t item);

typedef struct {
    oracle_item_fn fn;
    const void* args;
    int64_t items;
    atomic_llong next;
    atomic_int rc;
} oracle_farm_state;

static void* oracle_farm_worker(void* arg)
{
    oracle_farm_state* f = (oracle_farm_state*)arg;
    for (;;) {
        const int64_t i = atomic_fetch_add(&f->next, 1);
        if (i >= f->items || atomic_load(&f->rc) != 0)
            break;
        const int rc = f->fn(f->args, i);
        if (rc != 0) {
            int zero = 0;
            atomic_compare_exchange_strong(&f->rc, &zero, rc);
        }
    }
    return NULL;
}

static int oracle_farm(oracle_item_fn fn, const void* args, int64_t items, int threads)
{
    if (threads <= 1 || items <= 1) {
        for (int64_t i = 0; i < items; ++i) {
            const int rc = fn(args, i);
            if (rc != 0)
                return rc;
        }
        return 0;
    }
    if (threads > 256)
        threads = 256;
    oracle_farm_state f;
    f.fn = fn;
    f.args = args;
    f.items = items;
    atomic_init(&f.next, 0);
    atomic_init(&f.rc, 0);
    pthread_t tid[256];
    int started = 0;
    for (int t = 0; t < threads; ++t) {
        if (pthread_create(&tid[t], NULL, oracle_farm_worker, &f) != 0)
            break;
        ++started;
    }
    if (started == 0)
        oracle_farm_worker(&f);
    for (int t = 0; t < started; ++t)
        pthread_join(tid[t], NULL);
    return atomic_load(&f.rc);
}

/* -------------------------------------------- ragged forward and verify --- */

/*
 * Arguments of the [fwd] and [verify] walks.  All arrays contiguous:
 *   row_offsets [B+1], slot_idx [B], qkv [T, 2*nk*K + nv*V],
 *   decay, beta [T, nv], state [max_slots, nv, K, V], out [T, nv*V],
 *   ring [ring_rows, nk, ring_len, rec_stride] (verify only, else NULL),
 *   ring_slot_idx [B].
 * Verify ([verify] summary): same outputs as the forward; a row no longer than
 * ring_len writes one record per token and leaves the state alone; a longer
 * row writes no record and stores its state like the forward.
 */
typedef struct {
    int B, nv, nk, K, V;
    const uint32_t* row_offsets;
    const uint32_t* slot_idx;
    const float* qkv;
    const float* decay;
    const float* beta;
    int state_bf16;
    void* state;
    int64_t max_slots;
    float* out;
    float scale;
    int l2norm;
    void* ring;
    int ring_bf16;
    const uint32_t* ring_slot_idx;
    int64_t ring_rows;
    int ring_len;
    int64_t rec_stride;
} oracle_walk_args;

/* One work item of the walk: row b, value head hv (item = b * nv + hv). */
static int oracle_walk_item(const void* args, int64_t item)
{
    const oracle_walk_args* w = (const oracle_walk_args*)args;
    const int nv = w->nv, nk = w->nk, K = w->K, V = w->V;
    const int b = (int)(item / nv);
    const int hv = (int)(item % nv);
    const int G = nv / nk;
    const int64_t conv_dim = 2 * (int64_t)nk * K + (int64_t)nv * V;
    const int64_t kv = (int64_t)K * V;
    const uint32_t* row_offsets = w->row_offsets;
    float* out = w->out;
    void* ring = w->ring;
    const int ring_len = w->ring_len;

    const int64_t t0 = row_offsets[b], t1 = row_offsets[b + 1];
    const uint32_t slot = w->slot_idx[b];
    const int h = hv / G;
    const int m = hv % G;
    if (slot == ORACLE_PAD_SLOT) {
        for (int64_t t = t0; t < t1; ++t)
            for (int j = 0; j < V; ++j)
                out[t * nv * V + (int64_t)hv * V + j] = 0.0f;
        return 0;
    }
    if ((int64_t)slot >= w->max_slots)
        return -2;
    const int64_t soff = ((int64_t)slot * nv + hv) * kv;
    const int use_ring = ring != NULL && (t1 - t0) <= ring_len;
    const uint32_t rrow = ring ? w->ring_slot_idx[b] : 0;
    if (ring && use_ring && (int64_t)rrow >= w->ring_rows)
        return -2;

    float* S = (float*)malloc(sizeof(float) * (size_t)kv);
    float* qhat = (float*)malloc(sizeof(float) * (size_t)K);
    float* khat = (float*)malloc(sizeof(float) * (size_t)K);
    float* u = (float*)malloc(sizeof(float) * (size_t)V);
    oracle_load_block(w->state, w->state_bf16, soff, kv, S);
    for (int64_t t = t0; t < t1; ++t) {
        const float* row = w->qkv + t * conv_dim;
        oracle_packed_qk(row, nk, K, h, w->l2norm, qhat, khat);
        const float* v = row + 2 * (int64_t)nk * K + (int64_t)hv * V;
        const float a = w->decay[t * nv + hv];
        const float bt = w->beta[t * nv + hv];
        oracle_step(K, V, S, khat, qhat, v, a, &bt, 0, w->scale,
                    out + t * nv * V + (int64_t)hv * V, u);
        if (use_ring) {
            const int64_t rec = (((int64_t)rrow * nk + h) * ring_len + (t - t0)) * w->rec_stride;
            if (m == 0)
                for (int i = 0; i < K; ++i)
                    oracle_ring_put(ring, w->ring_bf16, rec + i, khat[i]);
            for (int j = 0; j < V; ++j)
                oracle_ring_put(ring, w->ring_bf16, rec + K + (int64_t)m * V + j, u[j]);
            oracle_ring_put(ring, w->ring_bf16, rec + K + (int64_t)G * V + m, a);
        }
    }
    if (t1 > t0 && !use_ring)
        oracle_store_block(w->state, w->state_bf16, soff, kv, S);
    free(S);
    free(qhat);
    free(khat);
    free(u);
    return 0;
}

static int oracle_walk(const oracle_walk_args* w, int threads)
{
    if (w->nk <= 0 || w->nv % w->nk != 0)
        return -1;
    return oracle_farm(oracle_walk_item, w, (int64_t)w->B * w->nv, threads);
}

/* [fwd]: slot-indexed ragged forward; the state of slot slot_idx[b] is read,
 * advanced over the row and written back in place.  threads > 1 spreads the
 * independent (row, value head) items over that many threads. */
int oracle_recurrence_fwd_threads(int B, int nv, int nk, int K, int V,
                                  const uint32_t* row_offsets, const uint32_t* slot_idx,
                                  const float* qkv, const float* decay, const float* beta,
                                  int state_bf16, void* state, int64_t max_slots, float* out,
                                  float scale, int l2norm, int threads)
{
    const oracle_walk_args w = {B, nv, nk, K, V, row_offsets, slot_idx, qkv, decay, beta,
                                state_bf16, state, max_slots, out, scale, l2norm,
                                NULL, 0, NULL, 0, 0, 0};
    return oracle_walk(&w, threads);
}

int oracle_recurrence_fwd(int B, int nv, int nk, int K, int V, const uint32_t* row_offsets,
                          const uint32_t* slot_idx, const float* qkv, const float* decay,
                          const float* beta, int state_bf16, void* state, int64_t max_slots,
                          float* out, float scale, int l2norm)
{
    return oracle_recurrence_fwd_threads(B, nv, nk, K, V, row_offsets, slot_idx, qkv, decay,
                                         beta, state_bf16, state, max_slots, out, scale, l2norm,
                                         1);
}

/* [verify]: the forward over a verify window, recording a float32 (or bf16)
 * ring. */
int oracle_recurrence_verify_ring_threads(int B, int nv, int nk, int K, int V,
                                          const uint32_t* row_offsets, const uint32_t* slot_idx,
                                          const float* qkv, const float* decay,
                                          const float* beta, int state_bf16, void* state,
                                          int64_t max_slots, float* out, float scale,
                                          int l2norm, void* ring, int ring_bf16,
                                          const uint32_t* ring_slot_idx, int64_t ring_rows,
                                          int ring_len, int64_t rec_stride, int threads)
{
    if (rec_stride < (int64_t)K + (int64_t)(nv / (nk > 0 ? nk : 1)) * (V + 1))
        return -1;
    const oracle_walk_args w = {B, nv, nk, K, V, row_offsets, slot_idx, qkv, decay, beta,
                                state_bf16, state, max_slots, out, scale, l2norm,
                                ring, ring_bf16, ring_slot_idx, ring_rows, ring_len, rec_stride};
    return oracle_walk(&w, threads);
}

int oracle_recurrence_verify_ring(int B, int nv, int nk, int K, int V,
                                  const uint32_t* row_offsets, const uint32_t* slot_idx,
                                  const float* qkv, const float* decay, const float* beta,
                                  int state_bf16, void* state, int64_t max_slots, float* out,
                                  float scale, int l2norm, void* ring, int ring_bf16,
                                  const uint32_t* ring_slot_idx, int64_t ring_rows, int ring_len,
                                  int64_t rec_stride)
{
    return oracle_recurrence_verify_ring_threads(B, nv, nk, K, V, row_offsets, slot_idx, qkv,
                                                 decay, beta, state_bf16, state, max_slots, out,
                                                 scale, l2norm, ring, ring_bf16, ring_slot_idx,
                                                 ring_rows, ring_len, rec_stride, 1);
}

/* [verify] (fold paragraphs): advance the live state of row b over its first
 * accepted[b] ring records.  A count above ring_len (a row that committed in
 * full during verify) or of zero leaves the state alone. */
int oracle_state_fold(int B, int nv, int nk, int K, int V, const uint32_t* slot_idx,
                      int state_bf16, void* state, int64_t max_slots, const void* ring,
                      int ring_bf16,
                      const uint32_t* ring_slot_idx, int64_t ring_rows, int ring_len,
                      int64_t rec_stride, const uint32_t* accepted)
{
    if (nk <= 0 || nv % nk != 0)
        return -1;
    const int G = nv / nk;
    const int64_t kv = (int64_t)K * V;
    float* S = (float*)malloc(sizeof(float) * (size_t)kv);
    for (int b = 0; b < B; ++b) {
        const uint32_t n = accepted[b];
        const uint32_t slot = slot_idx[b];
        if (n == 0 || n > (uint32_t)ring_len || slot == ORACLE_PAD_SLOT)
            continue;
        if ((int64_t)slot >= max_slots || (int64_t)ring_slot_idx[b] >= ring_rows) {
            free(S);
            return -2;
        }
        for (int hv = 0; hv < nv; ++hv) {
            const int h = hv / G, m = hv % G;
            const int64_t soff = ((int64_t)slot * nv + hv) * kv;
            oracle_load_block(state, state_bf16, soff, kv, S);
            for (uint32_t t = 0; t < n; ++t) {
                const int64_t rec =
                    (((int64_t)ring_slot_idx[b] * nk + h) * ring_len + t) * rec_stride;
                const float a = oracle_ring_get(ring, ring_bf16, rec + K + (int64_t)G * V + m);
                for (int i = 0; i < K; ++i)
                    for (int j = 0; j < V; ++j)
                        S[i * V + j] = a * S[i * V + j];
                for (int i = 0; i < K; ++i) {
                    const float khat = oracle_ring_get(ring, ring_bf16, rec + i);
                    for (int j = 0; j < V; ++j) {
                        const float u = oracle_ring_get(ring, ring_bf16, rec + K + (int64_t)m * V + j);
                        S[i * V + j] = S[i * V + j] + khat * u;
                    }
                }
            }
            oracle_store_block(state, state_bf16, soff, kv, S);
        }
    }
    free(S);
    return 0;
}

/* ----------------------------------------------------- fused update ------ */

/*
 * [gdp] fused_recurrent_gated_delta_rule_update, all arrays contiguous:
 *   q, k [B, T, H, K]; v, o [B, T, HV, V]; g [B, T, HV] log decays or NULL
 *   (no decay); beta [B, T, HV] or [B, T, HV, V] (beta_per_v) or NULL (1).
 *   cu_seqlens [N+1] or NULL: with it B must be 1 and sequence n spans
 *   [cu_seqlens[n], cu_seqlens[n+1]) of the T axis; without it N = B and every
 *   sequence has T tokens.
 *   state [num_slots, HV, K, V] with state_indices [N] (-1 = padding: zero
 *   output, nothing else touched), or NULL; then initial_state [N, HV, K, V]
 *   (NULL = zeros) seeds the walk and final_state [N, HV, K, V] (or NULL)
 *   receives the end state.
 *   intermediate [num_slots, int_tokens, HV, K, V] or NULL: snapshot i of
 *   a slot is written once (i+1)*steps_per_token steps of the sequence are
 *   done, i.e. when draft token i is complete; needs state.  All state-like buffers share one
 *   storage dtype (state_bf16).
 */
typedef struct {
    int T, H, HV, K, V;
    const float* q;
    const float* k;
    const float* v;
    const float* g;
    const float* beta;
    int beta_per_v;
    float scale;
    int l2norm;
    const int32_t* cu_seqlens;
    int state_bf16;
    void* state;
    int64_t num_slots;
    const int32_t* state_indices;
    const void* initial_state;
    void* final_state;
    void* intermediate;
    int64_t int_tokens;
    int steps_per_token;
    float* o;
} oracle_fused_args;

/* One work item: sequence n, value head hv (item = n * HV + hv). */
static int oracle_fused_item(const void* args, int64_t item)
{
    const oracle_fused_args* w = (const oracle_fused_args*)args;
    const int H = w->H, HV = w->HV, K = w->K, V = w->V;
    const int n = (int)(item / HV);
    const int hv = (int)(item % HV);
    const int G = HV / H;
    const int64_t kv = (int64_t)K * V;
    const float* q = w->q;
    const float* k = w->k;
    const float* v = w->v;
    const float* g = w->g;
    const float* beta = w->beta;
    const int beta_per_v = w->beta_per_v;
    void* state = w->state;
    const int state_bf16 = w->state_bf16;
    const void* initial_state = w->initial_state;
    void* final_state = w->final_state;
    void* intermediate = w->intermediate;
    const int64_t int_tokens = w->int_tokens;
    const int steps_per_token = w->steps_per_token;
    float* o = w->o;

    /* flat token range on the (B*T) axis */
    int64_t f0, f1;
    if (w->cu_seqlens) {
        f0 = w->cu_seqlens[n];
        f1 = w->cu_seqlens[n + 1];
    } else {
        f0 = (int64_t)n * w->T;
        f1 = f0 + w->T;
    }
    int32_t idx = w->state_indices ? w->state_indices[n] : n;
    const int h = hv / G;
    if (state && w->state_indices && idx < 0) {
        for (int64_t f = f0; f < f1; ++f)
            for (int j = 0; j < V; ++j)
                o[(f * HV + hv) * V + j] = 0.0f;
        return 0;
    }
    if (state && (int64_t)idx >= w->num_slots)
        return -2;

    float* S = (float*)malloc(sizeof(float) * (size_t)kv);
    float* qhat = (float*)malloc(sizeof(float) * (size_t)K);
    float* khat = (float*)malloc(sizeof(float) * (size_t)K);
    if (state)
        oracle_load_block(state, state_bf16, ((int64_t)idx * HV + hv) * kv, kv, S);
    else if (initial_state)
        oracle_load_block(initial_state, state_bf16, ((int64_t)n * HV + hv) * kv, kv, S);
    else
        for (int64_t e = 0; e < kv; ++e)
            S[e] = 0.0f;

    for (int64_t f = f0; f < f1; ++f) {
        const float* qt = q + (f * H + h) * K;
        const float* kt = k + (f * H + h) * K;
        if (w->l2norm) {
            oracle_l2norm(K, qt, qhat);
            oracle_l2norm(K, kt, khat);
        } else {
            for (int i = 0; i < K; ++i) {
                qhat[i] = qt[i];
                khat[i] = kt[i];
            }
        }
        const float a = g ? expf(g[f * HV + hv]) : 1.0f;
        float one = 1.0f;
        const float* bt = &one;
        int per_v = 0;
        if (beta) {
            bt = beta_per_v ? beta + (f * HV + hv) * V : beta + (f * HV + hv);
            per_v = beta_per_v;
        }
        oracle_step(K, V, S, khat, qhat, v + (f * HV + hv) * V, a, bt, per_v, w->scale,
                    o + (f * HV + hv) * V, NULL);
        const int64_t step = f - f0 + 1;
        if (intermediate && step % steps_per_token == 0) {
            const int64_t i = step / steps_per_token - 1;
            if (i < int_tokens)
                oracle_store_block(intermediate, state_bf16,
                                   (((int64_t)idx * int_tokens + i) * HV + hv) * kv, kv, S);
        }
    }
    if (state)
        oracle_store_block(state, state_bf16, ((int64_t)idx * HV + hv) * kv, kv, S);
    else if (final_state)
        oracle_store_block(final_state, state_bf16, ((int64_t)n * HV + hv) * kv, kv, S);
    free(S);
    free(qhat);
    free(khat);
    return 0;
}

int oracle_fused_recurrent_update_threads(int B, int T, int H, int HV, int K, int V,
                                          const float* q, const float* k, const float* v,
                                          const float* g, const float* beta, int beta_per_v,
                                          float scale, int l2norm, const int32_t* cu_seqlens,
                                          int N, int state_bf16, void* state, int64_t num_slots,
                                          const int32_t* state_indices,
                                          const void* initial_state, void* final_state,
                                          void* intermediate, int64_t int_tokens,
                                          int steps_per_token, float* o, int threads)
{
    if (H <= 0 || HV % H != 0)
        return -1;
    if (cu_seqlens && B != 1)
        return -1;
    if (!cu_seqlens)
        N = B;
    if (intermediate && (!state || steps_per_token < 1))
        return -1;
    const oracle_fused_args w = {T, H, HV, K, V, q, k, v, g, beta, beta_per_v, scale, l2norm,
                                 cu_seqlens, state_bf16, state, num_slots, state_indices,
                                 initial_state, final_state, intermediate, int_tokens,
                                 steps_per_token, o};
    return oracle_farm(oracle_fused_item, &w, (int64_t)N * HV, threads);
}

int oracle_fused_recurrent_update(int B, int T, int H, int HV, int K, int V, const float* q,
                                  const float* k, const float* v, const float* g,
                                  const float* beta, int beta_per_v, float scale, int l2norm,
                                  const int32_t* cu_seqlens, int N, int state_bf16, void* state,
                                  int64_t num_slots, const int32_t* state_indices,
                                  const void* initial_state, void* final_state,
                                  void* intermediate, int64_t int_tokens, int steps_per_token,
                                  float* o)
{
    return oracle_fused_recurrent_update_threads(B, T, H, HV, K, V, q, k, v, g, beta,
                                                 beta_per_v, scale, l2norm, cu_seqlens, N,
                                                 state_bf16, state, num_slots, state_indices,
                                                 initial_state, final_state, intermediate,
                                                 int_tokens, steps_per_token, o, 1);
}

/* [shape]: the forward's output is [total_seq_len, num_value_heads * V]. */
void oracle_fwd_output_shape(int64_t total_seq_len, int64_t nv, int64_t V, int64_t out[2])
{
    out[0] = total_seq_len;
    out[1] = nv * V;
}

/* ------------------------------------------------- snapshot rollback ------ */

/*
 * [gdp] update() parameters, intermediate_states: snapshot i of a slot holds
 * the state once draft token i is complete; a verifier that accepts a prefix
 * of the draft tokens restores the slot from the snapshot of the last one.
 * For request n with slot idx = state_indices[n] (>= 0) and accepted[n] = a
 * draft tokens, 1 <= a <= int_tokens: state[idx] <- intermediate[idx, a-1].
 * a == 0, a > int_tokens and padding requests (-1) leave the state alone (the
 * state before the first draft token is not among the snapshots).
 * state [num_slots, HV, K, V], intermediate [num_slots, int_tokens, HV, K, V],
 * both of one storage type (elem_size bytes per element).
 */
int oracle_snapshot_rollback(int N, int HV, int K, int V, int elem_size, void* state,
                             int64_t num_slots, const void* intermediate, int64_t int_tokens,
                             const int32_t* state_indices, const int32_t* accepted)
{
    const int64_t block = (int64_t)HV * K * V * elem_size;
    for (int n = 0; n < N; ++n) {
        const int32_t idx = state_indices[n];
        const int32_t a = accepted[n];
        if (idx < 0 || a < 1 || (int64_t)a > int_tokens)
            continue;
        if ((int64_t)idx >= num_slots)
            return -2;
        const char* src = (const char*)intermediate + ((int64_t)idx * int_tokens + (a - 1)) * block;
        char* dst = (char*)state + (int64_t)idx * block;
        for (int64_t b = 0; b < block; ++b)
            dst[b] = src[b];
    }
    return 0;
}

/* ---------------------------------------------- Pass-1 causal Conv1d ------ */

/*
 * [fwd] Args, qkv_conv_output: the recurrence consumes the output of a
 * Conv1d "Pass 1" that the pages name but do not specify.  Reading used here
 * (the plainest one the name and the packed layout support): a causal,
 * depthwise (one filter per channel) convolution along the token axis of each
 * ragged row, of width W, plus an optional per-channel bias, optionally
 * followed by SiLU, y * sigmoid(y).  Each row continues the history of its
 * slot: the W-1 inputs before the row's first token come from conv_state
 * (zeros when conv_state is NULL), and after the row the slot's conv_state
 * holds the last W-1 inputs of history ++ row.
 *
 *   x, out      [T, C] (out written for every token of every row)
 *   weight      [C, W]: tap j multiplies the input W-1-j tokens back
 *   bias        [C] or NULL
 *   conv_state  [num_slots, W-1, C] or NULL; entry i holds the input at
 *               relative position i - (W-1) before the row (i = W-2 is the
 *               most recent)
 *   slot_idx    [B] (0xFFFFFFFF = padding: zero output, nothing touched)
 *   row_offsets [B+1]
 * Rows of length 0 leave everything alone.
 */
int oracle_causal_conv1d(int B, int C, int W, const uint32_t* row_offsets,
                         const uint32_t* slot_idx, const float* x, const float* weight,
                         const float* bias, float* conv_state, int64_t num_slots, int silu,
                         float* out)
{
    const int H = W - 1;
    float* window = (float*)malloc(sizeof(float) * (size_t)W);
    for (int b = 0; b < B; ++b) {
        const int64_t t0 = row_offsets[b], t1 = row_offsets[b + 1];
        const uint32_t slot = slot_idx[b];
        if (slot == ORACLE_PAD_SLOT) {
            for (int64_t t = t0; t < t1; ++t)
                for (int c = 0; c < C; ++c)
                    out[t * C + c] = 0.0f;
            continue;
        }
        if (t1 <= t0)
            continue;
        if (conv_state && (int64_t)slot >= num_slots) {
            free(window);
            return -2;
        }
        for (int c = 0; c < C; ++c) {
            for (int64_t t = t0; t < t1; ++t) {
                /* window[j] = input at position t - (W-1) + j */
                for (int j = 0; j < W; ++j) {
                    const int64_t s = t - H + j;
                    if (s >= t0)
                        window[j] = x[s * C + c];
                    else if (conv_state)
                        window[j] = conv_state[((int64_t)slot * H + (H + (s - t0))) * C + c];
                    else
                        window[j] = 0.0f;
                }
                float y = bias ? bias[c] : 0.0f;
                for (int j = 0; j < W; ++j)
                    y = y + weight[(int64_t)c * W + j] * window[j];
                if (silu)
                    y = y / (1.0f + expf(-y));
                out[t * C + c] = y;
            }
        }
        if (conv_state) {
            /* new history: the last H inputs of old history ++ row */
            const int64_t L = t1 - t0;
            for (int c = 0; c < C; ++c) {
                float* hist = window; /* reuse: H <= W values */
                for (int i = 0; i < H; ++i) {
                    const int64_t s = t1 - H + i; /* absolute position */
                    if (s >= t0)
                        hist[i] = x[s * C + c];
                    else
                        hist[i] = conv_state[((int64_t)slot * H + (L + i)) * C + c];
                }
                for (int i = 0; i < H; ++i)
                    conv_state[((int64_t)slot * H + i) * C + c] = hist[i];
            }
        }
    }
    free(window);
    return 0;
}
