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

// R consecutive ring elements (float32 or bf16) widened to float.
template <int R>
__device__ __forceinline__ void load_run(const float* p, float (&out)[R]) {
    if constexpr (R % 4 == 0) {
#pragma unroll
        for (int i = 0; i < R; i += 4) load_cols<4>(p + i, out + i);
    } else {
        load_cols<R>(p, out);
    }
}
template <int R>
__device__ __forceinline__ void load_run(const uint16_t* p, float (&out)[R]) {
    if constexpr (R % 8 == 0) {
#pragma unroll
        for (int i = 0; i < R; i += 8) load_cols<8>(p + i, out + i);
    } else {
        load_cols<R>(p, out);
    }
}

template <int K, int CPL, int WPG, typename ST, typename RT>
__global__ void __launch_bounds__(WPG * 64) fold_kernel(const FoldParams p) {
    constexpr int V = K;
    constexpr int R = K / kRowGroups;
    constexpr int BV = kLanesPerRow * CPL;
    constexpr int TILES = V / BV;

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
    const int hv = h * p.G + m;
    const int j0 = vt * BV + vl * CPL;

    const uint32_t n = p.accepted[row];
    const uint32_t slot = p.slot_idx[row];
    if (n == 0 || n > static_cast<uint32_t>(p.ring_len) || slot == kPadSlot) return;

    ST* sp = static_cast<ST*>(p.state) + static_cast<int64_t>(slot) * p.st_slot +
             static_cast<int64_t>(hv) * p.st_head + j0;
    float S[R][CPL];
#pragma unroll
    for (int ri = 0; ri < R; ++ri) {
        RawCols<ST, CPL> raw;
        load_raw_cols<CPL>(sp + key_row<R>(kg, ri) * V, raw);
        widen_cols<CPL>(raw, S[ri]);
    }

    const RT* rec = static_cast<const RT*>(p.ring) +
                    static_cast<int64_t>(p.ring_idx[row]) * p.ring_row +
                    static_cast<int64_t>(h) * p.ring_head;
    float scale = 1.0f;
    for (uint32_t t = 0; t < n; ++t) {
        const RT* r = rec + static_cast<int64_t>(t) * p.ring_tok;
        float a;
        load_cols<1>(r + K + p.G * V + m, &a);
        float kr[R];
        load_run<R>(r + key_row<R>(kg, 0), kr);
        float u[CPL];
        load_cols<CPL>(r + K + m * V + j0, u);
        scale = decay_step<R, CPL>(S, scale * a);
        const float rho = __builtin_amdgcn_rcpf(scale);
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
            const float us = u[cc] * rho;
#pragma unroll
            for (int ri = 0; ri < R; ++ri) S[ri][cc] = __builtin_fmaf(kr[ri], us, S[ri][cc]);
        }
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
        case 128: return s.cpl == kFoldCpl ? launch_fold_wpg<128, kFoldCpl, ST>(p, s.wpg, stream) : hipErrorInvalidValue;
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
