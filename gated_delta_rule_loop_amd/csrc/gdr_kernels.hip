// gfx950 kernels of the gated delta rule library, part two: the fold of
// verify-ring records into the live state, the snapshot rollback copy and the
// host-side dispatch of every launch.  The recurrence kernels themselves are
// in gdr_device.h; their tables are compiled by gdr_rec_table.hip.
#include "gdr_device.h"

namespace gdr {

// Recurrence tables, one translation unit each (gdr_rec_table.hip).
extern template hipError_t launch_rec_table<float, uint16_t, kPlain>(const RecParams&,
                                                                  const LaunchShape&, hipStream_t);
extern template hipError_t launch_rec_table<float, uint16_t, kVerify>(const RecParams&,
                                                                  const LaunchShape&, hipStream_t);
extern template hipError_t launch_rec_table<float, uint16_t, kSnap>(const RecParams&,
                                                                  const LaunchShape&, hipStream_t);
extern template hipError_t launch_rec_table<float, uint16_t, kPlain | kBetaCols>(const RecParams&,
                                                                  const LaunchShape&, hipStream_t);
extern template hipError_t launch_rec_table<float, uint16_t, kSnap | kBetaCols>(const RecParams&,
                                                                  const LaunchShape&, hipStream_t);
extern template hipError_t launch_rec_table<float, float, kPlain>(const RecParams&,
                                                                  const LaunchShape&, hipStream_t);
extern template hipError_t launch_rec_table<float, float, kVerify>(const RecParams&,
                                                                  const LaunchShape&, hipStream_t);
extern template hipError_t launch_rec_table<float, float, kSnap>(const RecParams&,
                                                                  const LaunchShape&, hipStream_t);
extern template hipError_t launch_rec_table<float, float, kPlain | kBetaCols>(const RecParams&,
                                                                  const LaunchShape&, hipStream_t);
extern template hipError_t launch_rec_table<float, float, kSnap | kBetaCols>(const RecParams&,
                                                                  const LaunchShape&, hipStream_t);
extern template hipError_t launch_rec_table<uint16_t, uint16_t, kPlain>(const RecParams&,
                                                                  const LaunchShape&, hipStream_t);
extern template hipError_t launch_rec_table<uint16_t, uint16_t, kVerify>(const RecParams&,
                                                                  const LaunchShape&, hipStream_t);
extern template hipError_t launch_rec_table<uint16_t, uint16_t, kSnap>(const RecParams&,
                                                                  const LaunchShape&, hipStream_t);
extern template hipError_t launch_rec_table<uint16_t, uint16_t, kPlain | kBetaCols>(const RecParams&,
                                                                  const LaunchShape&, hipStream_t);
extern template hipError_t launch_rec_table<uint16_t, uint16_t, kSnap | kBetaCols>(const RecParams&,
                                                                  const LaunchShape&, hipStream_t);
extern template hipError_t launch_rec_table<uint16_t, float, kPlain>(const RecParams&,
                                                                  const LaunchShape&, hipStream_t);
extern template hipError_t launch_rec_table<uint16_t, float, kVerify>(const RecParams&,
                                                                  const LaunchShape&, hipStream_t);
extern template hipError_t launch_rec_table<uint16_t, float, kSnap>(const RecParams&,
                                                                  const LaunchShape&, hipStream_t);
extern template hipError_t launch_rec_table<uint16_t, float, kPlain | kBetaCols>(const RecParams&,
                                                                  const LaunchShape&, hipStream_t);
extern template hipError_t launch_rec_table<uint16_t, float, kSnap | kBetaCols>(const RecParams&,
                                                                  const LaunchShape&, hipStream_t);

namespace {

// ------------------------------------------------------------------- fold ---

// The ring records a workgroup folds are staged in LDS, kFoldStage tokens at
// a time, by loads issued together with the state loads: the token walk then
// reads LDS, so a wave waits for memory once rather than once per token.
// Staged token: the key row (padded per row group as stage_pos when the group
// holds a multiple of 4 rows), then u and the decay of each value head the
// workgroup covers.
template <int K, int HW>
struct FoldStage {
    static constexpr int R = K / kRowGroups;
    static constexpr bool kPad = R % 4 == 0;
    static constexpr int kK = kPad ? K + kRowGroups * 4 : K;   // staged key row
    static constexpr int kTok = kK + HW * K + ((HW + 3) & ~3);  // floats per token (V = K)
    __device__ static int kpos(int idx) { return kPad ? stage_pos<R>(idx) : idx; }
};

template <int K, int CPL, int WPG, typename ST, typename RT>
__global__ void __launch_bounds__(WPG * 64) fold_kernel(const FoldParams p) {
    constexpr int V = K;
    constexpr int R = K / kRowGroups;
    constexpr int BV = kLanesPerRow * CPL;
    constexpr int TILES = V / BV;
    constexpr int HW = WPG > TILES ? WPG / TILES : 1;  // value heads per workgroup
    using FS = FoldStage<K, HW>;
    constexpr int TCH = kFoldStage;
    constexpr int KV = K / 4, UV = V / 4;               // 4-element runs of k and of u
    constexpr int PER_TOK = KV + HW * UV + HW;          // loads per token (a: one each)
    constexpr int NT = WPG * 64;
    constexpr int ITEMS = (TCH * PER_TOK + NT - 1) / NT;
    __shared__ __attribute__((aligned(16))) float stage[TCH * FS::kTok];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int kg = lane >> 3;  // 8 consecutive lanes cover one contiguous row run
    const int vl = lane & 7;
    int blk = blockIdx.x;
    const int part = blk % p.parts;
    blk /= p.parts;
    const int h = blk % p.nk;
    const int row = blk / p.nk;
    const int unit = part * WPG + w;
    const int m = unit / TILES;
    const int vt = unit - m * TILES;
    const int m0 = (part * WPG) / TILES;  // first value head (within the key head) of the workgroup
    const int hv = h * p.G + m;
    const int j0 = vt * BV + vl * CPL;

    const uint32_t n = p.accepted[row];
    const uint32_t slot = p.slot_idx[row];
    if (n == 0 || n > static_cast<uint32_t>(p.ring_len) || slot == kPadSlot) return;

    ST* sp = static_cast<ST*>(p.state) + static_cast<int64_t>(slot) * p.st_slot +
             static_cast<int64_t>(hv) * p.st_head + j0;
    RawCols<ST, CPL> raw[R];
#pragma unroll
    for (int ri = 0; ri < R; ++ri) load_raw_cols<CPL>(sp + key_row<R>(kg, ri) * V, raw[ri]);

    const RT* rec = static_cast<const RT*>(p.ring) +
                    static_cast<int64_t>(p.ring_idx[row]) * p.ring_row +
                    static_cast<int64_t>(h) * p.ring_head;
    // Stage tokens [t0, t0 + cnt) of the ring into LDS.  The thread index is
    // re-read per stage so that the item addresses are not held across the
    // token walk.
    auto stage_in = [&](uint32_t t0, int cnt) {
        const int tid = fresh_lane<true>(static_cast<int>(threadIdx.x));
        constexpr int IB = ITEMS < 4 ? ITEMS : 4;  // items in flight per thread
#pragma unroll
        for (int b0 = 0; b0 < ITEMS; b0 += IB) {
            float buf[IB][4];
#pragma unroll
            for (int ib = 0; ib < IB; ++ib) {
                const int i = (b0 + ib) * NT + tid;
                const int tk = i / PER_TOK, e = i - tk * PER_TOK;
                if (b0 + ib < ITEMS && tk < cnt) {
                    const RT* r = rec + static_cast<int64_t>(t0 + tk) * p.ring_tok;
                    if (e < KV) {
                        load_cols<4>(r + 4 * e, buf[ib]);
                    } else if (e < KV + HW * UV) {
                        const int f = e - KV, hh = f / UV;
                        load_cols<4>(r + K + (m0 + hh) * V + 4 * (f - hh * UV), buf[ib]);
                    } else {
                        load_cols<1>(r + K + p.G * V + m0 + (e - KV - HW * UV), buf[ib]);
                    }
                }
            }
#pragma unroll
            for (int ib = 0; ib < IB; ++ib) {
                const int i = (b0 + ib) * NT + tid;
                const int tk = i / PER_TOK, e = i - tk * PER_TOK;
                if (b0 + ib < ITEMS && tk < cnt) {
                    float* d = stage + tk * FS::kTok;
                    if (e < KV) {
                        // a run of 4 stays inside one row group (R % 4 == 0 or no padding)
                        *reinterpret_cast<float4*>(d + FS::kpos(4 * e)) =
                            make_float4(buf[ib][0], buf[ib][1], buf[ib][2], buf[ib][3]);
                    } else if (e < KV + HW * UV) {
                        *reinterpret_cast<float4*>(d + FS::kK + 4 * (e - KV)) =
                            make_float4(buf[ib][0], buf[ib][1], buf[ib][2], buf[ib][3]);
                    } else {
                        d[FS::kK + HW * V + (e - KV - HW * UV)] = buf[ib][0];
                    }
                }
            }
        }
        __syncthreads();
    };
    const int um = m - m0;  // this wave's head among the staged ones
    const uint32_t tch = TCH;
    stage_in(0, static_cast<int>(min(n, tch)));
    float S[R][CPL];
#pragma unroll
    for (int ri = 0; ri < R; ++ri) widen_cols<CPL>(raw[ri], S[ri]);
    float scale = 1.0f;
    for (uint32_t t0 = 0;;) {
        const int cnt = static_cast<int>(min(n - t0, tch));
        for (int tk = 0; tk < cnt; ++tk) {
            const float* d = stage + tk * FS::kTok;
            const float a = d[FS::kK + HW * V + um];
            float kr[R];
            if constexpr (FS::kPad) {
                read_rows<R>(d, kg, kr);
            } else {
#pragma unroll
                for (int ri = 0; ri < R; ++ri) kr[ri] = d[kg * R + ri];
            }
            float u[CPL];
            load_cols<CPL>(d + FS::kK + um * V + j0, u);
            scale = decay_step<R, CPL>(S, scale * a);
            const float rho = __builtin_amdgcn_rcpf(scale);
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) {
                const float us = u[cc] * rho;
#pragma unroll
                for (int ri = 0; ri < R; ++ri) S[ri][cc] = __builtin_fmaf(kr[ri], us, S[ri][cc]);
            }
        }
        t0 += tch;
        if (t0 >= n) break;
        __syncthreads();  // every wave has read the stage
        stage_in(t0, static_cast<int>(min(n - t0, tch)));
    }
#pragma unroll
    for (int ri = 0; ri < R; ++ri) {
        float row[CPL];
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) row[cc] = scale * S[ri][cc];
        store_state_cols<CPL>(sp + key_row<R>(kg, ri) * V, row);
    }
}

// -------------------------------------------------------------- rollback ---

// A 16-byte vector as a native clang vector (kept in registers, unlike the
// HIP uint4 wrapper struct, which an unrolled copy left on the stack).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// state[slot, hv] <- intermediate[slot, a-1, hv]: a plain copy of one dense
// K x V block, 16 bytes per lane, kRollbackPerThread vectors in flight.
__global__ void __launch_bounds__(kRollbackThreads) rollback_kernel(const RollbackParams p) {
    const int chunk = blockIdx.x % p.chunks;
    const int rh = blockIdx.x / p.chunks;
    const int hv = rh % p.HV;
    const int row = rh / p.HV;
    const int32_t idx = p.idx[row];
    const int32_t a = p.accepted[row];
    if (idx < 0 || a < 1 || a > p.int_tokens) return;
    const u32x4* src = reinterpret_cast<const u32x4*>(
        static_cast<const char*>(p.inter) + idx * p.in_slot + static_cast<int64_t>(a - 1) * p.in_tok +
        hv * p.in_head);
    u32x4* dst = reinterpret_cast<u32x4*>(static_cast<char*>(p.state) + idx * p.st_slot +
                                          hv * p.st_head);
    const int64_t base = static_cast<int64_t>(chunk) * kRollbackThreads * kRollbackPerThread +
                         threadIdx.x;
    if (base + (kRollbackPerThread - 1) * kRollbackThreads < p.block16) {
        // whole chunk in range: all loads in flight before the first store
        u32x4 v[kRollbackPerThread];
#pragma unroll
        for (int j = 0; j < kRollbackPerThread; ++j) v[j] = state_ld<true>(src + base + j * kRollbackThreads);
#pragma unroll
        for (int j = 0; j < kRollbackPerThread; ++j) state_st<true>(v[j], dst + base + j * kRollbackThreads);
    } else {
        for (int64_t i = base; i < p.block16; i += kRollbackThreads) state_st<true>(state_ld<true>(src + i), dst + i);
    }
}
}  // namespace

hipError_t launch_rollback(const RollbackParams& p, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(p.rows) * p.HV * p.chunks);
    hipLaunchKernelGGL(rollback_kernel, grid, dim3(kRollbackThreads), 0, stream, p);
    return hipGetLastError();
}

// ------------------------------------------------------------- dispatch ---

template <typename WT, typename ST>
static hipError_t launch_rec_st(const RecParams& p, const LaunchShape& s, hipStream_t stream) {
    if (p.ring) {  // the packed verify has head-wise beta only
        if (p.beta_cols) return hipErrorInvalidValue;
        return launch_rec_table<WT, ST, kVerify>(p, s, stream);
    }
    if (p.beta_cols) {
        if (p.snap) return launch_rec_table<WT, ST, kSnap | kBetaCols>(p, s, stream);
        return launch_rec_table<WT, ST, kPlain | kBetaCols>(p, s, stream);
    }
    if (p.snap) return launch_rec_table<WT, ST, kSnap>(p, s, stream);
    return launch_rec_table<WT, ST, kPlain>(p, s, stream);
}

template <typename WT>
static hipError_t launch_rec_wt(const RecParams& p, const LaunchShape& s, StateType st,
                                hipStream_t stream) {
    return st == StateType::BF16 ? launch_rec_st<WT, uint16_t>(p, s, stream)
                                 : launch_rec_st<WT, float>(p, s, stream);
}

hipError_t launch_recurrence(const RecParams& p, const LaunchShape& s, StateType st,
                             bool work_bf16, hipStream_t stream) {
    return work_bf16 ? launch_rec_wt<uint16_t>(p, s, st, stream)
                     : launch_rec_wt<float>(p, s, st, stream);
}

template <int K, int CPL, typename ST, typename RT>
static hipError_t launch_fold_rt(const FoldParams& p, int wpg, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(p.rows) * p.nk * p.parts);
    switch (wpg) {
        case 1: hipLaunchKernelGGL((fold_kernel<K, CPL, 1, ST, RT>), grid, dim3(64), 0, stream, p); break;
        case 2: hipLaunchKernelGGL((fold_kernel<K, CPL, 2, ST, RT>), grid, dim3(128), 0, stream, p); break;
        case 4: hipLaunchKernelGGL((fold_kernel<K, CPL, 4, ST, RT>), grid, dim3(256), 0, stream, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int K, int CPL, typename ST>
static hipError_t launch_fold_wpg(const FoldParams& p, int wpg, hipStream_t stream) {
    return p.ring_bf16 ? launch_fold_rt<K, CPL, ST, uint16_t>(p, wpg, stream)
                       : launch_fold_rt<K, CPL, ST, float>(p, wpg, stream);
}

template <typename ST>
static hipError_t launch_fold_st(const FoldParams& p, const LaunchShape& s, hipStream_t stream) {
    switch (s.K) {
        case 128:
            if (p.ring_bf16)
                return s.cpl == kFoldCplBf16Ring
                           ? launch_fold_rt<128, kFoldCplBf16Ring, ST, uint16_t>(p, s.wpg, stream)
                           : hipErrorInvalidValue;
            return s.cpl == kFoldCpl ? launch_fold_rt<128, kFoldCpl, ST, float>(p, s.wpg, stream)
                                     : hipErrorInvalidValue;
        case 256: return s.cpl == 2 ? launch_fold_wpg<256, 2, ST>(p, s.wpg, stream) : hipErrorInvalidValue;
        case 64: return s.cpl == 8 ? launch_fold_wpg<64, 8, ST>(p, s.wpg, stream) : hipErrorInvalidValue;
        case 32: return s.cpl == 4 ? launch_fold_wpg<32, 4, ST>(p, s.wpg, stream) : hipErrorInvalidValue;
        case 16: return s.cpl == 2 ? launch_fold_wpg<16, 2, ST>(p, s.wpg, stream) : hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_fold(const FoldParams& p, const LaunchShape& s, StateType st,
                       hipStream_t stream) {
    return st == StateType::BF16 ? launch_fold_st<uint16_t>(p, s, stream)
                                 : launch_fold_st<float>(p, s, stream);
}

}  // namespace gdr
