// Internal launch parameters shared by the host entry points and the gfx950
// kernels of the gated delta rule library.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdr_fastdiv.h"

namespace gdr {

constexpr uint32_t kPadSlot = 0xFFFFFFFFu;


// One launch of the recurrence kernel.  All strides are in elements.
// A token tensor X of row r, sequence-local token t and head hd lives at
//   X + (offsets ? offsets[r] * x_tok : r * x_seq) + t * x_tok + hd * x_head.
struct RecParams {
    int32_t rows;        // batch rows (sequences)
    int32_t nv, nk, G;   // value heads, key heads, value heads per key head
    int32_t parts;       // workgroups per (row, key head)
    FastDiv div_parts, div_nk, div_row;  // by parts, nk and parts * nk
    int32_t dense_len;   // tokens per row when offsets == nullptr
    const uint32_t* offsets;

    // Per-token tensors, all of the work type (float32 or bf16).
    const void* q; int64_t q_seq, q_tok, q_head;
    const void* k; int64_t k_seq, k_tok, k_head;
    const void* v; int64_t v_seq, v_tok, v_head;
    const void* gate; int64_t g_seq, g_tok, g_head;    // nullptr: a = 1
    int32_t gate_is_log;                               // a = exp(gate)
    const void* beta; int64_t b_seq, b_tok, b_head;    // nullptr: beta = 1
    int32_t beta_cols;                                 // beta has a unit-stride V axis
    void* out; int64_t o_seq, o_tok, o_head;

    // State: slot = slot_idx[row] (nullptr: slot = row).  kPadSlot pads.
    const uint32_t* slot_idx;
    const void* src; int64_t src_slot, src_head; int32_t src_by_slot;  // nullptr: zeros
    void* dst; int64_t dst_slot, dst_head; int32_t dst_by_slot;        // nullptr: no store

    // Snapshots (fused update): entry i after (i+1)*spt steps, at dst slot.
    void* snap; int64_t snap_slot, snap_tok, snap_head; int32_t snap_count, spt;

    // Verify ring (float32, or bf16 when ring_bf16): rows with length <=
    // ring_len record and do not store.
    void* ring; const uint32_t* ring_idx;
    int64_t ring_row, ring_head, ring_tok; int32_t ring_len, ring_bf16;

    float scale;
    int32_t l2norm;
    int32_t order;   // 1: workgroups take the rows longest first (offsets, <= kOrderMaxRows rows)
};

// Longest-first row order: lengths are bucketed (kOrderBuckets buckets, exact
// below 32 tokens and four per octave above), and every workgroup ranks the
// rows itself, so it is offered for small batches only.
constexpr int kOrderBuckets = 64;
constexpr int kOrderMaxRows = 256;

struct FoldParams {
    int32_t rows, nv, nk, G, parts;
    const uint32_t* slot_idx;
    void* state; int64_t st_slot, st_head;
    const void* ring; const uint32_t* ring_idx;
    int64_t ring_row, ring_head, ring_tok; int32_t ring_len, ring_bf16;
    const uint32_t* accepted;
};

struct RollbackParams {
    int32_t rows, HV, chunks;  // workgroups per (request, head) = chunks
    const int32_t* idx;        // state_indices (-1 = padding)
    const int32_t* accepted;
    void* state; int64_t st_slot, st_head;                       // bytes
    const void* inter; int64_t in_slot, in_tok, in_head;         // bytes
    int32_t int_tokens;
    int64_t block16;           // 16-byte units per (slot, head) block
};

// Pass-1 causal depthwise Conv1d over ragged rows (strides in elements).
struct ConvParams {
    int32_t B, C, T, W;
    int32_t silu;
    const uint32_t* offsets;    // [B+1]
    const uint32_t* slot_idx;   // [B] or nullptr (slot = row); kPadSlot pads
    const void* x; int64_t x_tok;       // [T, C], work type
    void* out; int64_t o_tok;           // [T, C], work type
    const float* weight; int64_t w_chan; // [C, W]
    const float* bias;                  // [C] or nullptr
    void* state; int64_t st_slot, st_tok;  // [slots, W-1, C], work type, or nullptr
};

enum class StateType { F32 = 0, BF16 = 1 };

// Launch configuration picked by the host for one call.
struct LaunchShape {
    int K, V;       // key and value head dims
    int cpl;        // value columns per lane (8 lanes share one key-row group)
    int chunk;      // tokens staged per barrier
    int wpg;        // waves per workgroup
    bool kg_low;    // lane layout: row group in the low lane bits
};

// Host-side launchers (defined next to the kernels).  Return hipError_t.
hipError_t launch_recurrence(const RecParams& p, const LaunchShape& s, StateType st,
                             bool work_bf16, hipStream_t stream);
hipError_t launch_fold(const FoldParams& p, const LaunchShape& s, StateType st,
                       hipStream_t stream);
hipError_t launch_rollback(const RollbackParams& p, hipStream_t stream);
hipError_t launch_conv(const ConvParams& p, bool work_bf16, hipStream_t stream);
constexpr int kRollbackThreads = 256;
constexpr int kRollbackPerThread = 8;  // 16-byte vectors per thread

// Launch profiles at K = 128 (value columns per lane, tokens per stage, lane
// layout).  The reduction order does not depend on them, so they are free
// tuning choices: decode (about one token per row), tiny decode batches (at
// most 256 waves at the decode tiling), short windows (verify), the fused
// update on short rows (GDP decode, snapshot-heavy), long rows (prefill) and
// the fold.
constexpr int kDecodeCpl = 8;
constexpr int kTinyCpl = 2;
constexpr int kDecodeChunk = 1;
constexpr bool kDecodeKgLow = false;
constexpr int kShortCpl = 4;
constexpr int kShortChunk = 8;
constexpr bool kShortKgLow = false;
constexpr int kFusedCpl = 8;
constexpr int kFusedChunk = 4;
constexpr bool kFusedKgLow = false;
constexpr int kLongCpl = 2;
constexpr int kLongChunk = 32;
constexpr bool kLongKgLow = true;
constexpr int kFoldCpl = 4;         // float32 ring
constexpr int kFoldCplBf16Ring = 8; // bf16 ring
constexpr int kFoldStage = 8;       // ring tokens staged in LDS per fold pass

// Columns per wave for a given lanes-per-column setting.
constexpr int kLanesPerRow = 8;   // lanes that share one key-row group
constexpr int kRowGroups = 8;     // key-row groups per wave (64 / 8)

}  // namespace gdr
