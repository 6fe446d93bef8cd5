// gfx950 kernels of the Pass-1 causal Conv1d that produces the recurrence's
// packed qkv_conv_output (page "gated_delta_recurrence_fwd_gpu", Args: the input
// is the output of a first-pass convolution that the page names without
// specifying it).
//
// Reading implemented (the same as the CPU oracle's): a causal depthwise
// convolution of width W along the token axis of each ragged row, optional
// per-channel bias, optional SiLU; each row continues its slot's history of
// the W-1 previous inputs (conv_state [slots, W-1, C]) and leaves the last W-1
// inputs of history ++ row there.
//
// Two launches on the caller's stream.  conv_out_kernel: each thread owns 4
// adjacent channels (one 16-byte float32 or 8-byte bf16 access per token, so a
// wave reads 1 KiB of one token row) and a run of CH consecutive tokens, whose
// inputs it loads up front; it slides a window of the W-1 previous inputs in
// registers and refills it from the history or from x when it crosses into a
// new row.  conv_state_kernel then writes the new history of rows of two or
// more tokens; running it after the first launch is what keeps the in-place
// history update free of races (every output that reads the old history has
// been computed).  A one-token row (a decode step) has a single reader of its
// history, the thread of its token, which writes the new history itself, so a
// decode step reads the history once.  The work is a stream over x, out and
// the history: HBM-bound, no LDS.
#include "gdr_internal.h"

namespace gdr {
namespace {

constexpr int kConvThreads = 256;
constexpr int kConvVec = 4;  // channels per thread

__device__ __forceinline__ void load4(const float* p, float (&v)[4]) {
    const float4 w = *reinterpret_cast<const float4*>(p);
    v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
}
__device__ __forceinline__ void load4(const uint16_t* p, float (&v)[4]) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    v[0] = __uint_as_float(w.x << 16); v[1] = __uint_as_float(w.x & 0xFFFF0000u);
    v[2] = __uint_as_float(w.y << 16); v[3] = __uint_as_float(w.y & 0xFFFF0000u);
}
__device__ __forceinline__ void store4(float* p, const float (&v)[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
typedef __bf16 conv_bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    conv_bf16x2_t v = {(__bf16)lo, (__bf16)hi};  // round to nearest even
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ void store4(uint16_t* p, const float (&v)[4]) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack2(v[0], v[1]), pack2(v[2], v[3]));
}

// Row of token t: the last b in [0, B) with offsets[b] <= t.  Callers use it
// for offsets[0] <= t < offsets[B] only (and for a run start outside that
// range, whose tokens are then skipped).
__device__ __forceinline__ int row_of(const uint32_t* off, int B, uint32_t t) {
    int lo = 0, hi = B - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

template <int W, typename WT, int CH>
__global__ void __launch_bounds__(kConvThreads) conv_out_kernel(const ConvParams p) {
    constexpr int H = W - 1;
    const int c0 = (blockIdx.x * kConvThreads + threadIdx.x) * kConvVec;
    const int tstart = blockIdx.y * CH;
    if (c0 >= p.C || tstart >= p.T) return;
    const WT* x = static_cast<const WT*>(p.x) + c0;
    WT* out = static_cast<WT*>(p.out) + c0;

    // this run's inputs, loaded first (indices past the end clamped)
    float xs[CH][kConvVec];
#pragma unroll
    for (int i = 0; i < CH; ++i) load4(x + static_cast<int64_t>(min(tstart + i, p.T - 1)) * p.x_tok, xs[i]);

    float w[W][kConvVec], bias[kConvVec];
#pragma unroll
    for (int v = 0; v < kConvVec; ++v) {
#pragma unroll
        for (int j = 0; j < W; ++j) w[j][v] = p.weight[static_cast<int64_t>(c0 + v) * p.w_chan + j];
        bias[v] = p.bias ? p.bias[c0 + v] : 0.0f;
    }

    int b = row_of(p.offsets, p.B, static_cast<uint32_t>(tstart));
    int t0 = static_cast<int>(p.offsets[b]), t1 = static_cast<int>(p.offsets[b + 1]);
    // Tokens outside [offsets[0], offsets[B]) belong to no row: nothing is
    // read or written for them (x may be a padded token buffer).
    const int t_first = static_cast<int>(p.offsets[0]);
    const int t_end = min(p.T, static_cast<int>(p.offsets[p.B]));
    float win[H][kConvVec];  // win[i]: input at position t - H + i
    bool fresh = true;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int t = tstart + i;
        if (t >= t_end) break;
        if (t < t_first) continue;
        while (t >= t1) {  // next non-empty row (t < offsets[B], so b stays below B)
            ++b;
            t0 = t1;
            t1 = static_cast<int>(p.offsets[b + 1]);
            fresh = true;
        }
        const uint32_t slot = p.slot_idx ? p.slot_idx[b] : static_cast<uint32_t>(b);
        const bool pad = p.slot_idx != nullptr && slot == kPadSlot;
        if (fresh) {
            fresh = false;
#pragma unroll
            for (int k = 0; k < H; ++k) {
                const int s = t - H + k;
                if (s >= t0) {
                    load4(x + static_cast<int64_t>(s) * p.x_tok, win[k]);
                } else if (p.state && !pad) {
                    load4(static_cast<const WT*>(p.state) + static_cast<int64_t>(slot) * p.st_slot +
                              static_cast<int64_t>(H + s - t0) * p.st_tok + c0,
                          win[k]);
                } else {
#pragma unroll
                    for (int v = 0; v < kConvVec; ++v) win[k][v] = 0.0f;
                }
            }
        }
        float y[kConvVec];
#pragma unroll
        for (int v = 0; v < kConvVec; ++v) {
            float acc = bias[v];
#pragma unroll
            for (int j = 0; j < H; ++j) acc = __builtin_fmaf(w[j][v], win[j][v], acc);
            acc = __builtin_fmaf(w[H][v], xs[i][v], acc);
            if (p.silu) acc = acc / (1.0f + expf(-acc));
            y[v] = pad ? 0.0f : acc;
        }
        store4(out + static_cast<int64_t>(t) * p.o_tok, y);
#pragma unroll
        for (int v = 0; v < kConvVec; ++v) {
#pragma unroll
            for (int k = 0; k + 1 < H; ++k) win[k][v] = win[k + 1][v];
            win[H - 1][v] = xs[i][v];
        }
        // A one-token row's history was read by this thread alone, so it
        // writes the new one (the slid window) here and conv_state_kernel
        // skips the row.
        if (t1 - t0 == 1 && p.state && !pad) {
            WT* st = static_cast<WT*>(p.state) + static_cast<int64_t>(slot) * p.st_slot + c0;
#pragma unroll
            for (int k = 0; k < H; ++k) store4(st + static_cast<int64_t>(k) * p.st_tok, win[k]);
        }
    }
}

// New history of every non-padding row of two or more tokens (one-token rows
// are updated by conv_out_kernel): the last W-1 inputs of history ++ row.
// Runs after conv_out_kernel on the same stream.
template <int W, typename WT>
__global__ void __launch_bounds__(kConvThreads) conv_state_kernel(const ConvParams p) {
    constexpr int H = W - 1;
    const int c0 = (blockIdx.x * kConvThreads + threadIdx.x) * kConvVec;
    const int b = blockIdx.y;
    if (c0 >= p.C) return;
    const int t0 = static_cast<int>(p.offsets[b]), t1 = static_cast<int>(p.offsets[b + 1]);
    const int L = t1 - t0;
    const uint32_t slot = p.slot_idx ? p.slot_idx[b] : static_cast<uint32_t>(b);
    if (L <= 1 || (p.slot_idx != nullptr && slot == kPadSlot)) return;
    WT* st = static_cast<WT*>(p.state) + static_cast<int64_t>(slot) * p.st_slot + c0;
    const WT* x = static_cast<const WT*>(p.x) + c0;
    float old[H][kConvVec], nw[H][kConvVec];
#pragma unroll
    for (int i = 0; i < H; ++i) load4(st + static_cast<int64_t>(i) * p.st_tok, old[i]);
#pragma unroll
    for (int i = 0; i < H; ++i) {
        if (L + i < H) {  // still in the old history: entry L + i (selected, not indexed)
#pragma unroll
            for (int k = i + 1; k < H; ++k)
                if (k == L + i) {
#pragma unroll
                    for (int v = 0; v < kConvVec; ++v) nw[i][v] = old[k][v];
                }
        } else {
            load4(x + static_cast<int64_t>(t1 - H + i) * p.x_tok, nw[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < H; ++i) store4(st + static_cast<int64_t>(i) * p.st_tok, nw[i]);
}

template <int W, typename WT>
hipError_t launch_conv_w(const ConvParams& p, hipStream_t stream) {
    const unsigned cblocks = (p.C / kConvVec + kConvThreads - 1) / kConvThreads;
    // runs of 8 tokens when rows average 4 or more tokens, else one token
    if (p.T >= 4 * p.B) {
        const dim3 grid(cblocks, static_cast<unsigned>((int64_t{p.T} + 7) / 8));
        hipLaunchKernelGGL((conv_out_kernel<W, WT, 8>), grid, dim3(kConvThreads), 0, stream, p);
    } else {
        const dim3 grid(cblocks, p.T);
        hipLaunchKernelGGL((conv_out_kernel<W, WT, 1>), grid, dim3(kConvThreads), 0, stream, p);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !p.state) return e;
    hipLaunchKernelGGL((conv_state_kernel<W, WT>), dim3(cblocks, p.B), dim3(kConvThreads), 0,
                       stream, p);
    return hipGetLastError();
}

template <typename WT>
hipError_t launch_conv_wt(const ConvParams& p, hipStream_t stream) {
    switch (p.W) {
        case 2: return launch_conv_w<2, WT>(p, stream);
        case 3: return launch_conv_w<3, WT>(p, stream);
        case 4: return launch_conv_w<4, WT>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_conv(const ConvParams& p, bool work_bf16, hipStream_t stream) {
    return work_bf16 ? launch_conv_wt<uint16_t>(p, stream) : launch_conv_wt<float>(p, stream);
}

}  // namespace gdr
