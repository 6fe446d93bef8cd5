/*
 * gdr.h - C ABI of the MI355X (gfx950) gated delta rule recurrence library.
 *
 * The recurrence, per (sequence, value head), carries a K x V float32 state S
 * token by token:
 *     S <- a_t S;   u = beta_t (v_t - S^T k_t);   S <- S + k_t u^T;
 *     o_t = scale S^T q_t
 * with q_t, k_t optionally L2-normalised (x / sqrt(sum x^2 + GDR_L2NORM_EPS))
 * and scale defaulting to 1/sqrt(K).  Value head hv uses key head
 * hv / (num_value_heads / num_key_heads) (GQA).
 *
 * Conventions for every entry point
 *   - Tensors are described by gdr_tensor: data pointer, dtype, shape and
 *     strides in ELEMENTS.  All data pointers are DEVICE pointers owned by the
 *     caller; the library never allocates, frees or synchronises and keeps no
 *     pointer after returning.  A descriptor pointer of NULL, or one whose data
 *     is NULL, means an absent optional argument.  A required tensor with a
 *     zero extent may have NULL data (nothing is read or written through it;
 *     its strides are not checked).
 *   - Work is enqueued on the caller's HIP stream (hipStream_t passed as
 *     void*; NULL is the default stream).  Calls return once the work is
 *     enqueued.
 *   - Layout.  Tensors read or written with vector accesses need a unit
 *     innermost stride and a 16-byte aligned base: state pools, snapshots
 *     and initial/final states (each head's K x V block dense), rings,
 *     qkv_conv_output, recurrence_output, the fused update's q, k, v, o and
 *     per-column beta, and the Conv1d's x, out and history.  Their outer
 *     strides must keep 16-byte rows (multiples of 4 elements for float32
 *     and of 8 for bfloat16), except the Conv1d tensors (multiples of 4
 *     elements in either dtype).
 *     Per-token gates (decay, beta, g, head-wise beta) take any strides;
 *     index vectors of more than one element must be contiguous.
 *   - Return value: GDR_OK, or a negative GDR_ERR_* code with a message
 *     available from gdr_last_error_message() (thread-local).  Argument
 *     checks happen on the host before anything is enqueued; a failed check
 *     enqueues nothing.
 *   - Index contents (offsets, slots) are preconditions and are not checked
 *     on the device: offsets non-decreasing and ending at or before the
 *     token count, slots below the pool size and distinct within one call
 *     (two rows on one slot race).  gdr_check_indices checks them on the
 *     host, and gdr_set_debug_checks makes every call check its own.  Slot
 *     0xFFFFFFFF (-1 as int32) marks a padding row in every entry point: its
 *     output rows are written as +0.0 and no state, ring or snapshot memory
 *     is read or written for it.
 */
#ifndef GDR_H
#define GDR_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDR_OK 0
#define GDR_ERR_INVALID_ARG (-1) /* null, rank, shape or stride mismatch, or a
                                    batch whose launch grid would exceed 2^31-1
                                    workgroups */
#define GDR_ERR_UNSUPPORTED (-2) /* dtype, head dim or layout not built  */
#define GDR_ERR_HIP (-3)         /* the HIP runtime refused the launch    */

#define GDR_DTYPE_F32 0
#define GDR_DTYPE_BF16 1
#define GDR_DTYPE_U32 2
#define GDR_DTYPE_I32 3

#define GDR_MAX_DIMS 5

/* Flags */
#define GDR_FLAG_L2NORM_QK 1u /* L2-normalise q and k in the kernel */

/* L2 norm: x * (1 / sqrt(sum x^2 + GDR_L2NORM_EPS)). */
#define GDR_L2NORM_EPS 1e-6f

/* gdr_causal_conv1d flag: apply SiLU, y * sigmoid(y), to the conv output. */
#define GDR_FLAG_CONV_SILU 2u

/* Head dims built: K == V in {16, 32, 64, 128, 256}; the fused update also
 * takes (K, V) in {(64, 128), (128, 64), (128, 256), (256, 128)}. */
#define GDR_MAX_HEAD_DIM 256

typedef struct gdr_tensor {
    void* data;
    int32_t dtype; /* GDR_DTYPE_* */
    int32_t ndim;
    int64_t shape[GDR_MAX_DIMS];
    int64_t stride[GDR_MAX_DIMS]; /* in elements */
} gdr_tensor;

/*
 * gdr_recurrence_fwd - slot-indexed ragged forward.
 * Source: page "gated_delta_recurrence_fwd_gpu" (summary and Args); the
 * work dtype of the per-token tensors as on page
 * "gated_delta_recurrence_verify_ring_gpu" (Parameters, work_dtype).
 *
 * The per-token tensors (qkv_conv_output, decay_per_token, beta_per_token,
 * recurrence_output) share one work dtype, f32 or bf16; the arithmetic is
 * float32 either way (bf16 inputs widen exactly, bf16 outputs are rounded to
 * nearest even once).  2-D per-token tensors with vector accesses
 * (qkv_conv_output, recurrence_output) need 16-byte rows.
 *
 *   recurrence_output [T, nv*V] work  written for every token (out)
 *   recurrent_state   [slots, nv, K, V] bf16|f32, V contiguous, each head's
 *                     K x V block dense (in/out: the slot of each row is read
 *                     and written back in place; rows of length 0 are not
 *                     touched)
 *   slot_idx          [B] u32|i32     pool slot per row
 *   qkv_conv_output   [T, 2*nk*K + nv*V] work: q of key head h at channels
 *                     [h*K, (h+1)*K), k at nk*K + ..., v of value head hv at
 *                     2*nk*K + hv*V + ...
 *   decay_per_token   [T, nv] work    multiplicative decay a_t
 *   beta_per_token    [T, nv] work    beta gate
 *   input_row_offsets [B+1] u32|i32   row b spans [off[b], off[b+1]); tokens
 *                     outside [off[0], off[B]) belong to no row and their
 *                     output rows are not written
 *   scale             <= 0 or NaN selects 1/sqrt(K)
 *   flags             GDR_FLAG_L2NORM_QK (the page always normalises; pass it)
 */
int gdr_recurrence_fwd(int32_t num_value_heads, int32_t num_key_heads,
                       const gdr_tensor* recurrence_output, const gdr_tensor* recurrent_state,
                       const gdr_tensor* slot_idx, const gdr_tensor* qkv_conv_output,
                       const gdr_tensor* decay_per_token, const gdr_tensor* beta_per_token,
                       const gdr_tensor* input_row_offsets, float scale, uint32_t flags,
                       void* stream);

/*
 * gdr_recurrence_verify_ring - the forward over a speculative verify window
 * that records a per-token ring instead of writing the state back.
 * Source: page "gated_delta_recurrence_verify_ring_gpu" (summary, Parameters
 * ring_dtype and RING_LEN, Args ring / ring_slot_idx / ring_record_stride).
 *
 * Arguments as gdr_recurrence_fwd, plus
 *   ring              [ring_rows, nk, RING_LEN, record_stride] f32|bf16 (out);
 *                     the ring length is shape[2], record_stride is shape[3]
 *                     and must be >= gdr_ring_record_elements(nv/nk, K, V);
 *                     outer strides a multiple of 16 bytes
 *   ring_slot_idx     [B] u32|i32     ring row per batch row
 * Output equals gdr_recurrence_fwd's bit for bit.  A row of length
 * <= RING_LEN writes record [ring_row, key head, t] for each of its tokens t
 * and leaves recurrent_state untouched; a longer row writes no record and
 * stores its state exactly as the forward does (it commits in full).
 * Record layout (elements): [ k_hat (K) | u of value heads h*G+m, m < G (G*V)
 * | decay a of those heads (G) ] - the float32 operands of the state update
 * (rounded once to nearest-even bf16 in a bf16 ring), so the fold needs no
 * norm, exp or reduction.
 */
int gdr_recurrence_verify_ring(int32_t num_value_heads, int32_t num_key_heads,
                               const gdr_tensor* recurrence_output,
                               const gdr_tensor* recurrent_state, const gdr_tensor* slot_idx,
                               const gdr_tensor* qkv_conv_output,
                               const gdr_tensor* decay_per_token,
                               const gdr_tensor* beta_per_token,
                               const gdr_tensor* input_row_offsets, const gdr_tensor* ring,
                               const gdr_tensor* ring_slot_idx, float scale, uint32_t flags,
                               void* stream);

/*
 * gdr_state_fold - advance each row's live state over its accepted prefix
 * using the ring written by gdr_recurrence_verify_ring.
 * Source: page "gated_delta_recurrence_verify_ring_gpu" (the paragraphs on
 * the fold and on rows longer than RING_LEN; ring_dtype on bit-exactness).
 *
 *   recurrent_state   [slots, nv, K, V] bf16|f32 (in/out)
 *   slot_idx          [B] u32|i32
 *   ring              [ring_rows, nk, RING_LEN, record_stride] f32|bf16 (in)
 *   ring_slot_idx     [B] u32|i32
 *   accepted          [B] u32|i32 (device) accepted token count n of row b
 * n == 0 or n > RING_LEN leaves the row alone (a row longer than RING_LEN
 * already committed in verify: pass its full length).  Otherwise records
 * 0..n-1 are applied.  With a float32 ring the result equals
 * gdr_recurrence_fwd over the first n tokens bit for bit; a bf16 ring gives
 * the fold of the widened records, which differs from it by the records'
 * rounding.
 */
int gdr_state_fold(int32_t num_value_heads, int32_t num_key_heads,
                   const gdr_tensor* recurrent_state, const gdr_tensor* slot_idx,
                   const gdr_tensor* ring, const gdr_tensor* ring_slot_idx,
                   const gdr_tensor* accepted, void* stream);

/*
 * gdr_fused_recurrent_update - the recurrent step of the Gated Delta Rule /
 * Gated DeltaProduct decode path with a per-request state cache.
 * Source: page "core.ssm.ops.gdp.fused_recurrent"
 * (fused_recurrent_gated_delta_rule_update parameters; module summary on
 * Householder folding and intermediate states).
 *
 *   q, k              [B, T, H, K] work dtype: f32 or bf16, shared by q, k,
 *                     v, g, beta and o (float32 arithmetic either way)
 *   v                 [B, T, HV, V] work
 *   g                 [B, T, HV] work log decay (a = exp(g)), or absent (a = 1)
 *   beta              [B, T, HV] work, or [B, T, HV, V] work with unit stride
 *                     over V (one beta per value column), or absent (beta = 1)
 *   scale             <= 0 or NaN selects K^-0.5
 *   initial_state     [N, HV, K, V] bf16|f32 or absent (zeros); ignored when
 *                     state is given
 *   final_state       [N, HV, K, V] bf16|f32 (out) or absent; ignored when
 *                     state is given
 *   flags             GDR_FLAG_L2NORM_QK to normalise q and k
 *   cu_seqlens        [N+1] i32|u32 or absent: with it B must be 1 and
 *                     sequence n spans [cu[n], cu[n+1]) of the T axis;
 *                     without it N = B sequences of T tokens
 *   state             [S, HV, K, V] bf16|f32 cache, read and written in
 *                     place at state_indices (or at n when indices are absent)
 *   state_indices     [N] i32|u32, -1 = padding request (zero output, no
 *                     state or snapshot access)
 *   intermediate_states [S, T/steps_per_token, HV, K, V], same dtype as state,
 *                     or absent; needs state.  Snapshot i of a slot is
 *                     the state once (i+1)*steps_per_token steps of the
 *                     request are done (draft token i complete); steps past
 *                     shape[1] snapshots are not recorded.
 *   steps_per_token   >= 1
 *   o                 [B, T, HV, V] work (out)
 */
int gdr_fused_recurrent_update(const gdr_tensor* q, const gdr_tensor* k, const gdr_tensor* v,
                               const gdr_tensor* g, const gdr_tensor* beta, float scale,
                               const gdr_tensor* initial_state, const gdr_tensor* final_state,
                               uint32_t flags, const gdr_tensor* cu_seqlens,
                               const gdr_tensor* state, const gdr_tensor* state_indices,
                               const gdr_tensor* intermediate_states, int32_t steps_per_token,
                               const gdr_tensor* o, void* stream);

/*
 * gdr_snapshot_rollback - roll each request's cached state back to the
 * snapshot taken after its last accepted draft token.
 * Source: page "core.ssm.ops.gdp.fused_recurrent" (update() parameters,
 * intermediate_states: the snapshots exist so that a verifier that accepts
 * only some of the draft tokens can restore the state at the last accepted
 * one).
 *
 *   state               [S, HV, K, V] bf16|f32 cache (in/out)
 *   state_indices       [N] i32|u32 cache slot per request, -1 = padding
 *   intermediate_states [S, I, HV, K, V], same dtype as state (in)
 *   accepted            [N] i32|u32 (device): accepted draft tokens a of
 *                       request n
 * For 1 <= a <= I: state[slot] <- intermediate_states[slot, a-1], a copy of
 * the bits.  a == 0, a > I and padding requests leave the state untouched
 * (the state before the first draft token is not among the snapshots; a
 * caller that can accept zero drafts keeps its own copy).
 */
int gdr_snapshot_rollback(const gdr_tensor* state, const gdr_tensor* state_indices,
                          const gdr_tensor* intermediate_states, const gdr_tensor* accepted,
                          void* stream);

/*
 * gdr_causal_conv1d - the Conv1d "Pass 1" whose output is the forward's
 * qkv_conv_output.
 * Source: page "gated_delta_recurrence_fwd_gpu" (Args, qkv_conv_output: the
 * conv output from Pass 1, with q, k and v at fixed channel ranges).  The page
 * names the step only; implemented reading: a causal depthwise convolution of
 * width W along the token axis of each ragged row, plus an optional bias,
 * optionally followed by SiLU, where each row continues its slot's history.
 *
 *   out               [T, C] work dtype (f32|bf16) (out); must not alias x
 *   x                 [T, C] work dtype: the pre-conv projections; C a
 *                     multiple of 4, 16-byte aligned rows
 *   weight            [C, W] f32, W in {2, 3, 4}: tap j multiplies the input
 *                     W-1-j tokens back (unit stride over the taps)
 *   bias              [C] f32 or absent
 *   conv_state        [slots, W-1, C] work dtype (in/out) or absent (zero
 *                     history, nothing written): entry i is the input W-1-i
 *                     tokens before the row's first token; afterwards it holds
 *                     the last W-1 inputs of history ++ row
 *   slot_idx          [B] u32|i32 conv_state slot per row (absent: slot = row);
 *                     0xFFFFFFFF = padding (zero output, nothing touched)
 *   input_row_offsets [B+1] u32|i32 (B is shape[0] - 1); tokens of x
 *                     outside [off[0], off[B]) belong to no row: they are not
 *                     read and their output rows are not written
 *   flags             GDR_FLAG_CONV_SILU or 0
 * Rows of length 0 touch nothing.  Two kernel launches on `stream` (outputs,
 * then the history update).
 */
int gdr_causal_conv1d(const gdr_tensor* out, const gdr_tensor* x, const gdr_tensor* weight,
                      const gdr_tensor* bias, const gdr_tensor* conv_state,
                      const gdr_tensor* slot_idx, const gdr_tensor* input_row_offsets,
                      uint32_t flags, void* stream);

/*
 * gdr_fwd_output_shape - shape of recurrence_output for the given conv
 * output and state pool: {qkv.shape[0], state.shape[1] * state.shape[3]}.
 * Source: page "gated_delta_recurrence_fwd_shape".  Host only; reads shapes
 * only.  Returns GDR_OK or GDR_ERR_INVALID_ARG.
 */
int gdr_fwd_output_shape(const gdr_tensor* qkv_conv_output, const gdr_tensor* recurrent_state,
                         int64_t out_shape[2]);

/*
 * gdr_ring_record_elements - minimum record stride in elements for a key head
 * shared by `group` value heads: K + group * (V + 1).
 * Source: page "gated_delta_recurrence_verify_ring_gpu" (Args,
 * ring_record_stride).  Returns -1 for non-positive arguments.
 */
int64_t gdr_ring_record_elements(int32_t group, int32_t key_head_dim, int32_t value_head_dim);

/*
 * gdr_check_indices - host-side check of the index contents that every entry
 * point takes as preconditions (the kernels do not check them).  The arrays
 * are HOST memory; NULL skips that part of the check.
 *   rows          number of batch rows (or requests)
 *   row_offsets   [rows+1]: must not decrease, and must end at or before
 *                 total_tokens (input_row_offsets, or cu_seqlens as u32 bits)
 *   slots         [rows]: 0xFFFFFFFF (-1 as int32) is padding; any other
 *                 value must be below num_slots and used by one row only
 *   ring_idx      [rows] ring row of each row, checked for the rows that
 *                 use the ring: non-padding rows that record in a verify
 *                 (length <= ring_len; needs row_offsets) or, when accepted
 *                 is given, rows that a fold applies (0 < accepted <= ring_len).
 *                 Those must be below ring_rows and pairwise distinct.
 *   accepted      [rows] fold counts, or NULL for a verify
 * Returns GDR_OK, or GDR_ERR_INVALID_ARG with a message naming the first
 * offending row.  Host only; enqueues nothing.
 */
int gdr_check_indices(int64_t rows, const uint32_t* row_offsets, int64_t total_tokens,
                      const uint32_t* slots, int64_t num_slots, const uint32_t* ring_idx,
                      int64_t ring_rows, int64_t ring_len, const uint32_t* accepted);

/*
 * gdr_set_debug_checks - turn the index checks on (enable != 0) or off for
 * every later call in the process; returns the previous setting.  The
 * initial setting is on when the environment variable GDR_DEBUG_CHECK_SLOTS
 * holds a non-zero number.  With the checks on, each entry point copies its
 * index vectors to the host (this synchronises the caller's stream, so
 * checked calls cannot be captured into a HIP graph) and runs
 * gdr_check_indices on them before enqueueing anything; a failed check
 * returns GDR_ERR_INVALID_ARG and enqueues nothing.  A debugging aid for
 * callers that suspect duplicate or out-of-range slots; off by default.
 */
int gdr_set_debug_checks(int enable);

/* Message of the last failed call on this thread ("" when none). */
const char* gdr_last_error_message(void);

/* Library version string. */
const char* gdr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H */
