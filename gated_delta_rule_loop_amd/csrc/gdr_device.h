// gfx950 (CDNA4) kernels of the gated delta rule recurrence.
//
// Method (pages "gated_delta_recurrence_fwd_gpu", summary; and
// "core.ssm.ops.gdp.fused_recurrent", fused_recurrent_gated_delta_rule_fwd_kernel):
// per (sequence, value head) a K x V float32 state is carried token by token:
//     S <- a S;  u = beta (v - S^T k_hat);  S <- S + k_hat u^T;  o = scale S^T q_hat
//
// Work decomposition (ours, for 64-wide waves):
//   * one wave owns the full K extent of BV = 8*CPL contiguous value columns of
//     one value head: each lane belongs to one of 8 row groups kg and holds the
//     R = K/8 key rows [kg*R, kg*R + R) (key_row) of columns
//     [j0, j0 + CPL), j0 = 8*CPL*tile + CPL*(column chunk).  The state stays
//     in VGPRs for the whole row.
//   * the K-reduction of every column (S^T k_hat and S^T q_hat) is an in-lane
//     fused multiply-add chain over the lane's R rows in register order
//     followed by a butterfly over the 8 row groups (DPP and permlane adds).
//     This order depends on K only, never on CPL, the chunk size, the lane
//     layout or the workgroup shape, so every launch shape, the verify kernel
//     and the fold produce identical bits.
//   * a workgroup is WPG waves of one (row, key head); q/k of a chunk of C
//     tokens are normalised once per workgroup and staged in LDS together with
//     the chunk's v, decay and beta; the next chunk's global loads are issued
//     before the current chunk is processed.
//   * S^T k_hat of token t+1 is computed in the same register pass as the
//     read-out S^T q_hat of token t, so only one pass over the state is made
//     per token; decay is applied as r = a * (S^T k_hat) on the reduced value.
//   * no MFMA: the token-serial recurrence is not a dense contraction.
#pragma once

#include "gdr_internal.h"

namespace gdr {
namespace {

constexpr float kEps = 1e-6f;

// ------------------------------------------------------------ cross-lane ---

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// x[lane] + x[lane ^ 16], bit-identical in both lanes of the pair.
__device__ __forceinline__ float xor16_sum(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                              false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// x[lane] + x[lane ^ 32], bit-identical in both lanes of the pair.
__device__ __forceinline__ float xor32_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                              false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over the 8 key-row groups of a column, identical in all 8 lanes that
// hold them.  Both lane layouts (row group in the low or in the high three
// lane bits) add the groups as ((g0+g1)+(g2+g3)) + ((g4+g5)+(g6+g7)), so they
// give identical bits.
template <bool KG_LOW>
__device__ __forceinline__ float sum_row_groups(float x) {
    if constexpr (KG_LOW) {  // the 8 groups are the 8 lanes of one half-row
        x = x + dpp<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
        x = x + dpp<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
        x = x + dpp<0x141>(x);  // row_half_mirror: quads are uniform, pairs quad 0/1
    } else {                 // the groups are lanes l, l^8, ..., l^56
        x = x + dpp<0x128>(x);  // row_ror:8 is lane ^ 8 inside a 16-lane row
        x = xor16_sum(x);
        x = xor32_sum(x);
    }
    return x;
}

// Sum over aligned groups of N adjacent lanes (N = 2..64, a power of two),
// identical in every lane of a group: the pairs are added in the order
// lane^1, then quads, then half-rows (8), rows (16), 32 and 64 lanes.
template <int N>
__device__ __forceinline__ float sum_lanes(float x) {
    static_assert(N >= 2 && N <= 64 && (N & (N - 1)) == 0, "lane group");
    x = x + dpp<0xB1>(x);                     // quad_perm [1,0,3,2]: lane ^ 1
    if constexpr (N >= 4) x = x + dpp<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (N >= 8) x = x + dpp<0x141>(x);  // row_half_mirror: quads uniform, pairs quad 0/1
    if constexpr (N >= 16) x = x + dpp<0x140>(x); // row_mirror: half-rows uniform, pairs them
    if constexpr (N >= 32) x = xor16_sum(x);
    if constexpr (N >= 64) x = xor32_sum(x);
    return x;
}

// Several columns at once in the row-groups-high layout, same pairs and
// association as sum_row_groups<false> (so the same bits): after the DPP step
// each permlane swap carries two columns - a swap of (a, b) followed by one add
// leaves a's pair sums in some 16-lane rows and b's in the others.
__device__ __forceinline__ float pair16_sum(float a, float b) {
    // rows 0 and 2 get a[r] + a[r+1], rows 1 and 3 get b[r-1] + b[r]
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false,
                                              false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair32_sum(float a, float b) {
    // lanes 0-31 get a[lane] + a[lane + 32], lanes 32-63 get b[lane - 32] + b[lane]
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false,
                                              false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Column totals of CPL (2, 4 or 8) columns, spread over the 16-lane rows r:
// CPL 2: y[0] = column r & 1; CPL 4: y[0] = column r; CPL 8: y[0] = column r,
// y[1] = column 4 + r.
template <int CPL>
constexpr int kSpread = CPL == 8 ? 2 : 1;
template <int CPL>
__device__ __forceinline__ void sum_cols_spread(float (&x)[CPL], float (&y)[kSpread<CPL>]) {
    static_assert(CPL == 2 || CPL == 4 || CPL == 8, "spread reduction");
#pragma unroll
    for (int c = 0; c < CPL; ++c) x[c] = x[c] + dpp<0x128>(x[c]);  // lane ^ 8
    if constexpr (CPL == 2) {
        y[0] = xor32_sum(pair16_sum(x[0], x[1]));
    } else {
        y[0] = pair32_sum(pair16_sum(x[0], x[1]), pair16_sum(x[2], x[3]));
        if constexpr (CPL == 8)
            y[1] = pair32_sum(pair16_sum(x[4], x[5]), pair16_sum(x[6], x[7]));
    }
}

// Back from the spread form: every lane gets all CPL column totals.
template <int CPL>
__device__ __forceinline__ void spread_to_all(const float (&y)[kSpread<CPL>], float (&x)[CPL]) {
    auto both16 = [](float v, float& lo, float& hi) {  // rows [a b a b] -> [a..], [b..]
        auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
        lo = __uint_as_float(r[0]);
        hi = __uint_as_float(r[1]);
    };
    if constexpr (CPL == 2) {
        both16(y[0], x[0], x[1]);
    } else {
#pragma unroll
        for (int i = 0; i < kSpread<CPL>; ++i) {  // rows [a b c d] -> [a b a b], [c d c d]
            auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(y[i]),
                                                      __float_as_uint(y[i]), false, false);
            both16(__uint_as_float(r[0]), x[4 * i + 0], x[4 * i + 1]);
            both16(__uint_as_float(r[1]), x[4 * i + 2], x[4 * i + 3]);
        }
    }
}

// ------------------------------------------------------------- bf16 I/O ---

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t v = {(__bf16)lo, (__bf16)hi};  // round to nearest even
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <int CPL>
__device__ __forceinline__ void load_cols(const uint16_t* p, float* o) {
    if constexpr (CPL == 8) {
        const uint4 w = *reinterpret_cast<const uint4*>(p);
        o[0] = bf16_lo(w.x); o[1] = bf16_hi(w.x); o[2] = bf16_lo(w.y); o[3] = bf16_hi(w.y);
        o[4] = bf16_lo(w.z); o[5] = bf16_hi(w.z); o[6] = bf16_lo(w.w); o[7] = bf16_hi(w.w);
    } else if constexpr (CPL == 4) {
        const uint2 w = *reinterpret_cast<const uint2*>(p);
        o[0] = bf16_lo(w.x); o[1] = bf16_hi(w.x); o[2] = bf16_lo(w.y); o[3] = bf16_hi(w.y);
    } else if constexpr (CPL == 2) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
        o[0] = bf16_lo(w); o[1] = bf16_hi(w);
    } else {
        o[0] = __uint_as_float(static_cast<uint32_t>(*p) << 16);
    }
}

template <int CPL>
__device__ __forceinline__ void store_cols(uint16_t* p, const float* s) {
    if constexpr (CPL == 8) {
        uint4 w;
        w.x = pack_bf16x2(s[0], s[1]); w.y = pack_bf16x2(s[2], s[3]);
        w.z = pack_bf16x2(s[4], s[5]); w.w = pack_bf16x2(s[6], s[7]);
        *reinterpret_cast<uint4*>(p) = w;
    } else if constexpr (CPL == 4) {
        uint2 w;
        w.x = pack_bf16x2(s[0], s[1]); w.y = pack_bf16x2(s[2], s[3]);
        *reinterpret_cast<uint2*>(p) = w;
    } else if constexpr (CPL == 2) {
        *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(s[0], s[1]);
    } else {
        *p = static_cast<uint16_t>(pack_bf16x2(s[0], 0.0f) & 0xFFFFu);
    }
}

template <int CPL>
__device__ __forceinline__ void load_cols(const float* p, float* o) {
    if constexpr (CPL % 4 == 0) {
#pragma unroll
        for (int i = 0; i < CPL; i += 4) {
            const float4 w = *reinterpret_cast<const float4*>(p + i);
            o[i] = w.x; o[i + 1] = w.y; o[i + 2] = w.z; o[i + 3] = w.w;
        }
    } else if constexpr (CPL == 2) {
        const float2 w = *reinterpret_cast<const float2*>(p);
        o[0] = w.x; o[1] = w.y;
    } else {
        o[0] = *p;
    }
}

template <int CPL>
__device__ __forceinline__ void store_cols(float* p, const float* s) {
    if constexpr (CPL % 4 == 0) {
#pragma unroll
        for (int i = 0; i < CPL; i += 4)
            *reinterpret_cast<float4*>(p + i) = make_float4(s[i], s[i + 1], s[i + 2], s[i + 3]);
    } else if constexpr (CPL == 2) {
        *reinterpret_cast<float2*>(p) = make_float2(s[0], s[1]);
    } else {
        *p = s[0];
    }
}

// Raw state columns, widened only where first used, so that the wait for a
// state load can sit after the work that does not need it: bf16 pairs stay
// packed in dwords; float values need no conversion.
template <typename ST, int CPL>
struct RawCols {
    float v[CPL];
};
template <int CPL>
struct RawCols<uint16_t, CPL> {
    uint32_t v[(CPL + 1) / 2];
};

// State blocks are read once and written once per call.  Where one lane's
// access is 16 bytes, 8 lanes cover whole 128-byte lines and the accesses are
// non-temporal (streamed); narrower accesses leave each line to two waves,
// which rely on the cache to merge the halves, so they stay ordinary
// (measured: non-temporal 8-byte state accesses slowed the decode step by 20%,
// 16-byte ones sped the snapshot-heavy fused update up by 9%).
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <bool NT, typename T>
__device__ __forceinline__ T state_ld(const T* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    return *p;
}
template <bool NT, typename T>
__device__ __forceinline__ void state_st(T v, T* p) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

template <int CPL>
__device__ __forceinline__ void load_raw_cols(const float* p, RawCols<float, CPL>& r) {
    if constexpr (CPL % 4 == 0) {
#pragma unroll
        for (int i = 0; i < CPL; i += 4) {
            const f32x4_t w = state_ld<true>(reinterpret_cast<const f32x4_t*>(p + i));
            r.v[i] = w.x; r.v[i + 1] = w.y; r.v[i + 2] = w.z; r.v[i + 3] = w.w;
        }
    } else if constexpr (CPL == 2) {
        const f32x2_t w = state_ld<false>(reinterpret_cast<const f32x2_t*>(p));
        r.v[0] = w.x; r.v[1] = w.y;
    } else {
        r.v[0] = state_ld<false>(p);
    }
}
template <int CPL>
__device__ __forceinline__ void load_raw_cols(const uint16_t* p, RawCols<uint16_t, CPL>& r) {
    if constexpr (CPL == 8) {
        const u32x4_t w = state_ld<true>(reinterpret_cast<const u32x4_t*>(p));
        r.v[0] = w.x; r.v[1] = w.y; r.v[2] = w.z; r.v[3] = w.w;
    } else if constexpr (CPL == 4) {
        const u32x2_t w = state_ld<false>(reinterpret_cast<const u32x2_t*>(p));
        r.v[0] = w.x; r.v[1] = w.y;
    } else if constexpr (CPL == 2) {
        r.v[0] = state_ld<false>(reinterpret_cast<const uint32_t*>(p));
    } else {
        r.v[0] = state_ld<false>(p);
    }
}

// A state row fragment: CPL values stored (bf16 rounded to nearest even).
template <int CPL>
__device__ __forceinline__ void store_state_cols(float* p, const float* s) {
    if constexpr (CPL % 4 == 0) {
#pragma unroll
        for (int i = 0; i < CPL; i += 4)
            state_st<true>(f32x4_t{s[i], s[i + 1], s[i + 2], s[i + 3]},
                           reinterpret_cast<f32x4_t*>(p + i));
    } else if constexpr (CPL == 2) {
        state_st<false>(f32x2_t{s[0], s[1]}, reinterpret_cast<f32x2_t*>(p));
    } else {
        state_st<false>(s[0], p);
    }
}
template <int CPL>
__device__ __forceinline__ void store_state_cols(uint16_t* p, const float* s) {
    if constexpr (CPL == 8) {
        state_st<true>(u32x4_t{pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3]),
                               pack_bf16x2(s[4], s[5]), pack_bf16x2(s[6], s[7])},
                       reinterpret_cast<u32x4_t*>(p));
    } else if constexpr (CPL == 4) {
        state_st<false>(u32x2_t{pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3])},
                        reinterpret_cast<u32x2_t*>(p));
    } else if constexpr (CPL == 2) {
        state_st<false>(pack_bf16x2(s[0], s[1]), reinterpret_cast<uint32_t*>(p));
    } else {
        store_cols<1>(p, s);
    }
}
template <int CPL>
__device__ __forceinline__ void widen_cols(const RawCols<float, CPL>& r, float* o) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) o[c] = r.v[c];
}
template <int CPL>
__device__ __forceinline__ void widen_cols(const RawCols<uint16_t, CPL>& r, float* o) {
    if constexpr (CPL == 1) {
        o[0] = __uint_as_float(r.v[0] << 16);
    } else {
#pragma unroll
        for (int j = 0; j < CPL / 2; ++j) {
            o[2 * j] = bf16_lo(r.v[j]);
            o[2 * j + 1] = bf16_hi(r.v[j]);
        }
    }
}

// The lane index as a value the compiler may not hoist (when HIDE): staging
// code derives addresses from it, and computing them where they are used
// (once per stage) keeps them out of the registers that the token loop
// needs.  The short-row shapes, whose token loop fills the register budget,
// and the fold's record staging ask for it.
template <bool HIDE>
__device__ __forceinline__ int fresh_lane(int lane) {
    if constexpr (HIDE) asm volatile("" : "+v"(lane));
    return lane;
}

// x / d for x < 2^31 (see FastDiv).
__device__ __forceinline__ int fdiv(int x, FastDiv f) {
    const uint32_t u = static_cast<uint32_t>(x);
    return static_cast<int>((__umulhi(u, f.mul) + u) >> f.shift);
}

// ---------------------------------------------------- per-lane arithmetic ---

// The state of one (row, value head) is held as scale * S: a token's decay
// multiplies only the scalar (cn = scale * a), and the rank-1 write becomes
// S += k_hat (u / cn)^T, one fused multiply-add per element.  When cn leaves
// [2^-64, 2^64] (a zero decay included) the scale is folded into the registers
// and reset to 1.  The forward, the verify and the fold run this same scalar
// sequence from the same decays, so their states stay bit-identical.
constexpr uint32_t kScaleLoBits = 0x1F800000u;  // 2^-64
constexpr uint32_t kScaleHiBits = 0x5F800000u;  // 2^64

// cn in [2^-64, 2^64], by one unsigned compare: positive floats order as their
// bit patterns, and zero, negative values and NaN all fall outside.
__device__ __forceinline__ bool scale_in_range(float cn) {
    return __float_as_uint(cn) - kScaleLoBits <= kScaleHiBits - kScaleLoBits;
}

template <int R, int CPL>
__device__ __forceinline__ float decay_step(float (&S)[R][CPL], float cn) {
    if (__builtin_expect(scale_in_range(cn), 1)) return cn;
#pragma unroll
    for (int ri = 0; ri < R; ++ri)
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) S[ri][cc] = cn * S[ri][cc];
    return 1.0f;
}

// out[c] = sum_ri S[ri][c] * vec[ri], ascending ri, fused multiply-adds.
template <int R, int CPL>
__device__ __forceinline__ void dot_rows(const float (&S)[R][CPL], const float (&vec)[R],
                                         float (&out)[CPL]) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        float acc = S[0][c] * vec[0];
#pragma unroll
        for (int ri = 1; ri < R; ++ri) acc = __builtin_fmaf(S[ri][c], vec[ri], acc);
        out[c] = acc;
    }
}

// Key rows of a lane: row group kg (of 8) holds the R = K/8 consecutive key
// rows kg*R + ri.  Every kernel (forward, verify, fold) uses this one mapping,
// so their reduction orders stay identical.  (Interleaving the groups, row
// ri*8 + kg, was measured slower for the decode step and the fold.)
template <int R>
__device__ __forceinline__ int key_row(int kg, int ri) { return kg * R + ri; }

// A staged K-vector in LDS: row group kg's R values at kg*(R + 4), 4 floats
// of padding after each group so the 8 groups hit different banks.
template <int R>
__device__ __forceinline__ int stage_pos(int idx) { return idx + (idx / R) * 4; }

template <int R>
__device__ __forceinline__ void read_rows(const float* vec, int kg, float (&out)[R]) {
    const float* src = vec + kg * (R + 4);
    if constexpr (R % 4 == 0) {
#pragma unroll
        for (int i = 0; i < R; i += 4) {
            const float4 w = *reinterpret_cast<const float4*>(src + i);
            out[i] = w.x; out[i + 1] = w.y; out[i + 2] = w.z; out[i + 3] = w.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < R; ++i) out[i] = src[i];
    }
}

// ------------------------------------------------------------- recurrence ---

// Zeros read in place of the state rows when there is no source state.
__device__ __attribute__((aligned(16))) float kZeroRow[16];

// Kernel modes: kPlain, kVerify or kSnap, plus the kBetaCols bit when beta
// carries one value per value column.
enum : int { kPlain = 0, kVerify = 1, kSnap = 2, kBetaCols = 4 };

// One ring element: float32, or bf16 rounded to nearest even.
__device__ __forceinline__ void ring_put(const RecParams& p, int64_t i, float x) {
    if (p.ring_bf16)
        store_cols<1>(static_cast<uint16_t*>(p.ring) + i, &x);
    else
        static_cast<float*>(p.ring)[i] = x;
}

// N consecutive ring elements (16-byte aligned runs: N float32 or N bf16).
template <int N>
__device__ __forceinline__ void ring_put_run(const RecParams& p, int64_t i, const float (&x)[N]) {
    if (p.ring_bf16) {
        uint16_t* r = static_cast<uint16_t*>(p.ring) + i;
        if constexpr (N % 8 == 0) {
#pragma unroll
            for (int j = 0; j < N; j += 8)
                store_cols<8>(r + j, x + j);
        } else {
            store_cols<N>(r, x);
        }
    } else {
        float* r = static_cast<float*>(p.ring) + i;
        if constexpr (N % 4 == 0) {
#pragma unroll
            for (int j = 0; j < N; j += 4)
                store_cols<4>(r + j, x + j);
        } else {
            store_cols<N>(r, x);
        }
    }
}

// One work item: value columns [j0, j0 + CPL) of every key row, for one value
// head of one row, resolved once per item.
struct Item {
    int row, h, part, m, vt, hv, j0, L;
    int64_t rq, rk, rv, rg, rb, ro;
    uint32_t slot;
    bool pad, record;
};

// One element of a per-token tensor (float32, or bf16 bits widened exactly).
__device__ __forceinline__ float load1(const float* p) { return *p; }
__device__ __forceinline__ float load1(const uint16_t* p) {
    return __uint_as_float(static_cast<uint32_t>(*p) << 16);
}

// The same in two steps: the raw element (bf16 bits zero-extended, held in a
// float register), then its value.  Staged loads keep the raw form until
// their first arithmetic use, so no conversion forces an early wait.
__device__ __forceinline__ float load_raw(const float* p) { return *p; }
__device__ __forceinline__ float load_raw(const uint16_t* p) {
    return __uint_as_float(static_cast<uint32_t>(*p));
}
template <typename WT>
__device__ __forceinline__ float widen_raw(float raw) {
    if constexpr (sizeof(WT) == 2) return __uint_as_float(__float_as_uint(raw) << 16);
    return raw;
}

// N consecutive elements of a per-token tensor as loaded: float values, or
// bf16 bits packed two per dword (widened after the wait, see load_raw).
template <typename WT, int N>
struct RawVec {
    float v[N];
};
template <int N>
struct RawVec<uint16_t, N> {
    uint32_t v[(N + 1) / 2];
};

// N consecutive elements with the widest aligned vector loads (every caller's
// runs are aligned to their size).
template <int N>
__device__ __forceinline__ void load_vec(const float* p, RawVec<float, N>& r) {
    static_assert(N == 2 || N % 4 == 0, "float runs of 2 or 4k");
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N; i += 4) {
            const float4 w = *reinterpret_cast<const float4*>(p + i);
            r.v[i] = w.x; r.v[i + 1] = w.y; r.v[i + 2] = w.z; r.v[i + 3] = w.w;
        }
    } else {
        const float2 w = *reinterpret_cast<const float2*>(p);
        r.v[0] = w.x; r.v[1] = w.y;
    }
}
template <int N>
__device__ __forceinline__ void load_vec(const uint16_t* p, RawVec<uint16_t, N>& r) {
    static_assert(N == 2 || N == 4 || N % 8 == 0, "bf16 runs of 2, 4 or 8k");
    if constexpr (N % 8 == 0) {
#pragma unroll
        for (int i = 0; i < N / 2; i += 4) {
            const uint4 w = *reinterpret_cast<const uint4*>(p + 2 * i);
            r.v[i] = w.x; r.v[i + 1] = w.y; r.v[i + 2] = w.z; r.v[i + 3] = w.w;
        }
    } else if constexpr (N == 4) {
        const uint2 w = *reinterpret_cast<const uint2*>(p);
        r.v[0] = w.x; r.v[1] = w.y;
    } else {
        r.v[0] = *reinterpret_cast<const uint32_t*>(p);
    }
}
template <int N>
__device__ __forceinline__ void widen_vec(const RawVec<float, N>& r, float (&o)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) o[i] = r.v[i];
}
template <int N>
__device__ __forceinline__ void widen_vec(const RawVec<uint16_t, N>& r, float (&o)[N]) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
        o[2 * i] = bf16_lo(r.v[i]);
        o[2 * i + 1] = bf16_hi(r.v[i]);
    }
}
// N consecutive floats to LDS (16-byte stores where N allows; the callers'
// offsets keep them aligned).
template <int N>
__device__ __forceinline__ void lds_put(float* dst, const float (&x)[N]) {
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N; i += 4)
            *reinterpret_cast<float4*>(dst + i) = make_float4(x[i], x[i + 1], x[i + 2], x[i + 3]);
    } else if constexpr (N == 2) {
        *reinterpret_cast<float2*>(dst) = make_float2(x[0], x[1]);
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) dst[i] = x[i];
    }
}

// ST: state storage type; WT: per-token input/output type (float, or
// uint16_t holding bf16 bits).  Arithmetic is float32 either way.
template <int K, int V, int CPL, int C, int WPG, typename ST, bool KG_LOW, typename WT>
struct Rec {
    static constexpr int R = K / kRowGroups;
    static constexpr int BV = kLanesPerRow * CPL;
    static constexpr int TILES = V / BV;
    static constexpr int KP = K + 4 * kRowGroups;      // padded staged vector
    // L2 norms.  A token's q (or k) is split into NCH chunks of 4 elements;
    // a lane sums the squares of its chunk in element order, and the chunk
    // sums of a token are added by sum_lanes<NCH> - an order that depends on
    // K only, so every launch shape normalises identically.  A norm job is one
    // wave's worth of (token, tensor) units, lane = NCH * unit + chunk with
    // unit = 2 * token + (0 for k, 1 for q); the stage's jobs are spread over
    // the waves.
    // multi-token stages in the row-groups-high layout: the token loop uses
    // nearly the whole register budget (see fresh_lane)
    static constexpr bool kTightRegs = C > 1 && !KG_LOW;
    static constexpr int NCH = K / 4;                         // chunks per vector
    static constexpr int UPJ = 64 / NCH;                      // units per job
    static constexpr int NJOB = (2 * C + UPJ - 1) / UPJ;      // jobs per stage
    // One-token stages: every wave normalises the token itself into its own
    // copy of the staged k_hat and q_hat, so a wave needs no other wave's
    // work and the workgroup needs no barrier (see stage_sync).
    static constexpr bool kPrivStage = C == 1;
    static constexpr int JPW = kPrivStage ? NJOB : (NJOB + WPG - 1) / WPG;  // jobs per wave
    static constexpr int NKQ = kPrivStage ? WPG : 1;          // copies of k_hat, q_hat
    static_assert(K % 4 == 0 && NCH <= 64, "norm chunks");
    static constexpr int VTOT = C * BV;                // v floats per wave per chunk
    static constexpr int VPL = VTOT >= 64 ? VTOT / 64 : 1;
    static_assert(R >= 2 && TILES >= 1 && V % BV == 0, "tile shape");
    static_assert(VTOT < 64 || VTOT % 64 == 0, "v staging");
    static_assert(C <= 64, "gate staging uses one lane per token");

    // LDS: two chunk buffers of [NKQ x (k_hat C x KP | q_hat*scale C x KP) |
    // v | a | beta | per-column beta (kBetaCols only)]; wave w reads the
    // k_hat/q_hat copy at kq(w).
    static constexpr int OFF_K = 0;
    static constexpr int OFF_Q = C * KP;
    static constexpr int OFF_V = 2 * C * KP * NKQ;
    __device__ static int kq(int w) { return kPrivStage ? w * 2 * C * KP : 0; }
    static constexpr int OFF_A = OFF_V + WPG * VTOT;
    static constexpr int OFF_B = OFF_A + WPG * C;
    static constexpr int OFF_BV = (OFF_B + WPG * C + 3) / 4 * 4;
    template <bool BC>
    static constexpr int buf() { return BC ? OFF_BV + WPG * VTOT : OFF_BV; }

    struct Stage {
        RawVec<WT, 4> qk[JPW];
        float v[VPL], bv[VPL], a, b;
    };

    // Lane = 8 * column chunk + row group (KG_LOW) or 8 * row group + column
    // chunk.  The first keeps each reduction inside a DPP half-row; the second
    // keeps 8 consecutive lanes on one contiguous run of a state row.
    __device__ static int row_group(int lane) { return KG_LOW ? (lane & 7) : (lane >> 3); }
    __device__ static int col_chunk(int lane) { return KG_LOW ? (lane >> 3) : (lane & 7); }

    __device__ static Item item(const RecParams& p, int idx, int w, int lane) {
        Item it;
        const int blk = fdiv(idx, p.div_parts);
        it.part = idx - blk * p.parts;
        it.row = fdiv(blk, p.div_nk);
        it.h = blk - it.row * p.nk;
        const int unit = it.part * WPG + w;
        it.m = unit / TILES;
        it.vt = unit - it.m * TILES;
        it.hv = it.h * p.G + it.m;
        it.j0 = it.vt * BV + col_chunk(lane) * CPL;
        if (p.offsets) {
            const int64_t t0 = p.offsets[it.row];
            it.L = static_cast<int>(static_cast<int64_t>(p.offsets[it.row + 1]) - t0);
            it.rq = t0 * p.q_tok; it.rk = t0 * p.k_tok; it.rv = t0 * p.v_tok;
            it.rg = t0 * p.g_tok; it.rb = t0 * p.b_tok; it.ro = t0 * p.o_tok;
        } else {
            const int64_t r = it.row;
            it.L = p.dense_len;
            it.rq = r * p.q_seq; it.rk = r * p.k_seq; it.rv = r * p.v_seq;
            it.rg = r * p.g_seq; it.rb = r * p.b_seq; it.ro = r * p.o_seq;
        }
        it.slot = p.slot_idx ? p.slot_idx[it.row] : static_cast<uint32_t>(it.row);
        it.pad = p.slot_idx != nullptr && it.slot == kPadSlot;
        it.record = p.ring != nullptr && it.L <= p.ring_len;
        return it;
    }

    __device__ static WT* out_ptr(const RecParams& p, const Item& it) {
        return static_cast<WT*>(p.out) + it.ro + static_cast<int64_t>(it.hv) * p.o_head + it.j0;
    }

    __device__ static const ST* src_ptr(const RecParams& p, const Item& it) {
        const int64_t sel = p.src_by_slot ? static_cast<int64_t>(it.slot) : it.row;
        return static_cast<const ST*>(p.src) + sel * p.src_slot +
               static_cast<int64_t>(it.hv) * p.src_head + it.j0;
    }

    // Padding request: +0.0 output for every token, nothing else.
    __device__ static void zero_output(const RecParams& p, const Item& it, int lane) {
        if (row_group(lane) != 0) return;
        float z[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) z[c] = 0.0f;
        WT* outp = out_ptr(p, it);
        for (int t = 0; t < it.L; ++t) store_cols<CPL>(outp + t * p.o_tok, z);
    }

    // The lane's state rows as loaded (see RawCols).
    struct RawState {
        RawCols<ST, CPL> row[R];
    };

    // Without a source state every row is read from kZeroRow (row stride 0),
    // so the loads are unconditional and one wait covers them on every path.
    __device__ static void load_state(const RecParams& p, const Item& it, int kg, RawState& rs) {
        static_assert(CPL * sizeof(ST) <= sizeof(kZeroRow), "zero row");
        const bool has = p.src != nullptr;
        const ST* sp = has ? src_ptr(p, it) : reinterpret_cast<const ST*>(kZeroRow);
        const int row_stride = has ? V : 0;
#pragma unroll
        for (int ri = 0; ri < R; ++ri)
            load_raw_cols<CPL>(sp + key_row<R>(kg, ri) * row_stride, rs.row[ri]);
    }

    __device__ static void widen_state(const RawState& rs, float (&S)[R][CPL]) {
#pragma unroll
        for (int ri = 0; ri < R; ++ri) widen_cols<CPL>(rs.row[ri], S[ri]);
    }

    // Stores the state scale * S.
    __device__ static void store_tile(ST* base, int kg, float scale, const float (&S)[R][CPL]) {
#pragma unroll
        for (int ri = 0; ri < R; ++ri) {
            float row[CPL];
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) row[cc] = scale * S[ri][cc];
            store_state_cols<CPL>(base + key_row<R>(kg, ri) * V, row);
        }
    }

    __device__ static void store_state(const RecParams& p, const Item& it, int kg, float scale,
                                       const float (&S)[R][CPL]) {
        if (!p.dst || it.record) return;
        const int64_t sel = p.dst_by_slot ? static_cast<int64_t>(it.slot) : it.row;
        store_tile(static_cast<ST*>(p.dst) + sel * p.dst_slot +
                       static_cast<int64_t>(it.hv) * p.dst_head + it.j0,
                   kg, scale, S);
    }

    // The raw form (see load_raw) of 1.0.
    __device__ static float raw_one() {
        if constexpr (sizeof(WT) == 2) return __uint_as_float(0x3F80u);
        return 1.0f;
    }

    // v, or the per-column beta, of a chunk: VPL consecutive elements per
    // lane of the wave's C x BV block (one vector load).  Lanes past the block
    // or the row re-read a valid vector; those values are never read from
    // the stage (the token loop stops at the row's end).
    __device__ static void load_block(const WT* base, int64_t tok, int L, int tc, int lane,
                                      float (&dst)[VPL]) {
        const int flat = min(lane * VPL, VTOT - VPL);
        const int tau = flat / BV;
        const int col = flat - tau * BV;
        load_cols<VPL>(base + min(tc + tau, L - 1) * tok + col, dst);
    }

    // Global loads of chunk c of an item into registers.  Each load is
    // unconditional - an index past the row's end, the stage or the head dim
    // is clamped to a valid element - and nothing here depends on a loaded
    // value, so a stage's loads issue back to back and retire under a single
    // wait in commit_stage.  Values loaded for positions past the row or the
    // stage are never read.  The decay is kept raw (exp is applied in
    // commit_stage).
    template <bool BC>
    __device__ static void load_stage(const RecParams& p, const Item& it, int c, Stage& s,
                                      int w, int lane) {
        const int tc = c * C;
        const int last = it.L - 1;
        lane = fresh_lane<kTightRegs>(lane);
        const int chunk = lane % NCH;
#pragma unroll
        for (int i = 0; i < JPW; ++i) {
            const int job = kPrivStage ? i : w + i * WPG;  // wave-uniform
            if (job >= NJOB) break;
            const int unit = job * UPJ + lane / NCH;
            const int tau = unit >> 1;
            const int64_t tl = min(tc + tau, last);
            // Lanes of units past the stage or the row load the row's last
            // token instead; their results stay in their own lanes and are
            // never written.
            const WT* src = (unit & 1)
                                ? static_cast<const WT*>(p.q) + it.rq + tl * p.q_tok + it.h * p.q_head
                                : static_cast<const WT*>(p.k) + it.rk + tl * p.k_tok + it.h * p.k_head;
            load_vec<4>(src + chunk * 4, s.qk[i]);
        }
        load_block(static_cast<const WT*>(p.v) + it.rv + it.hv * p.v_head + it.vt * BV, p.v_tok,
                   it.L, tc, lane, s.v);
        if constexpr (BC)
            load_block(static_cast<const WT*>(p.beta) + it.rb + it.hv * p.b_head + it.vt * BV,
                       p.b_tok, it.L, tc, lane, s.bv);
        const int64_t tl = min(tc + min(lane, C - 1), last);
        // raw gates; an absent gate stages the raw form of 1 (of 0 for a log
        // decay, exp(0) = 1)
        s.a = p.gate_is_log ? 0.0f : raw_one();
        s.b = raw_one();
        if (p.gate)
            s.a = load_raw(static_cast<const WT*>(p.gate) + it.rg + tl * p.g_tok + it.hv * p.g_head);
        if (!BC && p.beta)
            s.b = load_raw(static_cast<const WT*>(p.beta) + it.rb + tl * p.b_tok + it.hv * p.b_head);
    }

    // Norms of the staged tokens, then k_hat, q_hat*scale, v and gates to LDS.
    // The first part of a (row, key head) also writes k_hat to the ring.
    template <bool BC>
    __device__ static void commit_stage(const RecParams& p, const Item& it, int c,
                                        const Stage& s, float* B, int w, int lane) {
        const int tc = c * C;
        const int64_t rec = it.record ? static_cast<int64_t>(p.ring_idx[it.row]) * p.ring_row +
                                            static_cast<int64_t>(it.h) * p.ring_head
                                      : 0;
        lane = fresh_lane<kTightRegs>(lane);
        const int chunk = lane % NCH;
#pragma unroll
        for (int i = 0; i < JPW; ++i) {
            const int job = kPrivStage ? i : w + i * WPG;  // wave-uniform
            // tokens past the row's end are never read from the stage
            if (job >= NJOB || tc + (job * UPJ) / 2 >= it.L) break;
            const int unit = job * UPJ + lane / NCH;
            const bool is_q = unit & 1;
            const int tau = unit >> 1;
            float x[4];
            widen_vec(s.qk[i], x);
            float f = is_q ? p.scale : 1.0f;
            if (p.l2norm) {
                float ss = x[0] * x[0];
#pragma unroll
                for (int e = 1; e < 4; ++e) ss = __builtin_fmaf(x[e], x[e], ss);
                ss = sum_lanes<NCH>(ss);
                const float r = rsqrtf(ss + kEps);
                f = is_q ? r * p.scale : r;
            }
            if (tau < C) {
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = x[e] * f;
                float* dst = B + kq(w) + (is_q ? OFF_Q : OFF_K) + tau * KP;
                if constexpr (R % 4 == 0) {
                    lds_put<4>(dst + stage_pos<R>(chunk * 4), x);
                } else {  // R == 2: the chunk spans two row groups
#pragma unroll
                    for (int e = 0; e < 4; ++e) dst[stage_pos<R>(chunk * 4 + e)] = x[e];
                }
                if (!is_q && it.record && it.part == 0 && (!kPrivStage || w == 0) &&
                    tc + tau < it.L)
                    ring_put_run<4>(p, rec + (tc + tau) * p.ring_tok + chunk * 4, x);
            }
        }
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int flat = lane * VPL + i;
            if (flat < VTOT) B[OFF_V + w * VTOT + flat] = s.v[i];
            if (BC && flat < VTOT) B[OFF_BV + w * VTOT + flat] = s.bv[i];
        }
        if (lane < C) {
            const float a = widen_raw<WT>(s.a);
            B[OFF_A + w * C + lane] = p.gate && p.gate_is_log ? expf(a) : a;
            B[OFF_B + w * C + lane] = widen_raw<WT>(s.b);
        }
    }

    // Column totals of a lane's CPL columns in every lane: through the spread
    // form in the row-groups-high layout (two columns per permlane swap),
    // column by column otherwise.  Both give the bits of sum_row_groups.
    // (Multi-token stages only: the one-token decode stage is bound by HBM and
    // measured a little faster column by column.)
    static constexpr bool kSpreadOut = !KG_LOW && C > 1 && (CPL == 2 || CPL == 4 || CPL == 8);
    __device__ static void sum_cols_all(float (&x)[CPL]) {
        if constexpr (kSpreadOut) {
            float y[kSpread<CPL>];
            sum_cols_spread<CPL>(x, y);
            spread_to_all<CPL>(y, x);
        } else {
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) x[cc] = sum_row_groups<KG_LOW>(x[cc]);
        }
    }

    // The tokens of chunk c, staged in B.  The state before the chunk is
    // scale * S; both are updated (see decay_step for the representation).
    // REC: record the ring for rows that fit it (verify); SNAP: store snapshots.
    template <bool REC, bool SNAP, bool BC>
    __device__ static void run_chunk(const RecParams& p, const Item& it, int c, const float* B,
                                     float (&S)[R][CPL], float& scale, int w, int lane) {
        const int kg = row_group(lane);
        const int vc = col_chunk(lane) * CPL;
        const int tc = c * C;
        // Tokens of this chunk; made a scalar for the multi-token loops (the
        // one-token decode stage measured a little faster without)
        const int Lc = C > 1 ? __builtin_amdgcn_readfirstlane(min(C, it.L - tc)) : min(C, it.L - tc);
        WT* outp = out_ptr(p, it) + static_cast<int64_t>(tc) * p.o_tok;
        int64_t rec = 0;  // ring element offset of this token's record
        if (REC && it.record)
            rec = static_cast<int64_t>(p.ring_idx[it.row]) * p.ring_row +
                  static_cast<int64_t>(it.h) * p.ring_head + static_cast<int64_t>(tc) * p.ring_tok;
        ST* snap = nullptr;
        int snap_left = 0;
        if constexpr (SNAP) {  // steps until the next snapshot, and its entry
            const int done = tc % p.spt;
            snap_left = p.spt - done;
            snap = static_cast<ST*>(p.snap) + static_cast<int64_t>(it.slot) * p.snap_slot +
                   static_cast<int64_t>(tc / p.spt) * p.snap_tok +
                   static_cast<int64_t>(it.hv) * p.snap_head + it.j0;
        }
        int snap_i = SNAP ? tc / p.spt : 0;

        // In the spread form (multi-token stages, row groups high) the
        // retrieval stays spread: this lane holds the totals of columns
        // vc + scol(i), computes u and u / scale for those columns only, and
        // broadcasts u / scale to the CPL columns it updates.  The same
        // operations on the same values per column as the column-by-column
        // path, so the same bits.
        const int r16 = lane >> 4;
        auto scol = [&](int i) { return (CPL == 2 ? (r16 & 1) : r16) + 4 * i; };
        const bool spread_lead = (lane & 8) == 0 && (CPL != 2 || lane < 32);
        const float* KQ = B + kq(w);  // this wave's k_hat / q_hat copy
        float kr[R];
        read_rows<R>(KQ + OFF_K, kg, kr);
        float x[CPL];                 // S^T k_hat of the current token, before the scale
        float xs[kSpread<CPL>];       // the same, spread (kSpreadOut)
        dot_rows<R, CPL>(S, kr, x);
        if constexpr (kSpreadOut) sum_cols_spread<CPL>(x, xs);
        else sum_cols_all(x);

        for (int tau = 0; tau < Lc; ++tau) {
            const float a = B[OFF_A + w * C + tau];
            const float b = BC ? 1.0f : B[OFF_B + w * C + tau];
            // r = S_{t-1}^T k_hat with this token's decay: (scale * a) * x
            const float cn = scale * a;
            float u[CPL];                 // column-by-column path
            float us[CPL];                // u / scale for the lane's columns
            float u_s[kSpread<CPL>];      // spread path: u of the spread columns
            if constexpr (kSpreadOut) {
#pragma unroll
                for (int i = 0; i < kSpread<CPL>; ++i) {
                    const int cc = scol(i);
                    const float vv = B[OFF_V + w * VTOT + tau * BV + vc + cc];
                    const float be = BC ? B[OFF_BV + w * VTOT + tau * BV + vc + cc] : b;
                    u_s[i] = be * (vv - cn * xs[i]);
                }
            } else {
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc) {
                    const float vv = B[OFF_V + w * VTOT + tau * BV + vc + cc];
                    const float be = BC ? B[OFF_BV + w * VTOT + tau * BV + vc + cc] : b;
                    u[cc] = be * (vv - cn * x[cc]);
                }
            }
            scale = decay_step<R, CPL>(S, cn);
            const float rho = __builtin_amdgcn_rcpf(scale);
            if constexpr (kSpreadOut) {
                float us_s[kSpread<CPL>];
#pragma unroll
                for (int i = 0; i < kSpread<CPL>; ++i) us_s[i] = u_s[i] * rho;
                spread_to_all<CPL>(us_s, us);
            } else {
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc) us[cc] = u[cc] * rho;
            }
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) {
#pragma unroll
                for (int ri = 0; ri < R; ++ri) S[ri][cc] = __builtin_fmaf(kr[ri], us[cc], S[ri][cc]);
            }

            float qr[R];
            read_rows<R>(KQ + OFF_Q + tau * KP, kg, qr);
            float o[CPL];
            dot_rows<R, CPL>(S, qr, o);
            if (C > 1 && tau + 1 < Lc) {
                read_rows<R>(KQ + OFF_K + (tau + 1) * KP, kg, kr);
                dot_rows<R, CPL>(S, kr, x);
                if constexpr (kSpreadOut) sum_cols_spread<CPL>(x, xs);
                else sum_cols_all(x);
            }
            if constexpr (kSpreadOut) {
                // totals spread over the rows: lanes of even row groups store
                // their row's column(s)
                float y[kSpread<CPL>];
                sum_cols_spread<CPL>(o, y);
                if (spread_lead) {
#pragma unroll
                    for (int i = 0; i < kSpread<CPL>; ++i) {
                        const float val = scale * y[i];
                        store_cols<1>(outp + scol(i), &val);
                    }
                }
            } else {
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc) o[cc] = scale * sum_row_groups<KG_LOW>(o[cc]);
                // Every lane holds its columns' totals.  With the row groups in
                // the low lane bits the 8 lanes of a column store the same bits
                // to the same address, which spares the long-row loop a lane
                // mask and its branches.
                if (KG_LOW || kg == 0) store_cols<CPL>(outp, o);
            }
            outp += p.o_tok;
            if (REC && it.record) {
                const int64_t ru = rec + K + it.m * V + it.j0;
                if constexpr (kSpreadOut) {  // u of the spread columns
                    if (spread_lead) {
#pragma unroll
                        for (int i = 0; i < kSpread<CPL>; ++i) ring_put(p, ru + scol(i), u_s[i]);
                    }
                } else if (kg == 0) {
                    if (p.ring_bf16)
                        store_cols<CPL>(static_cast<uint16_t*>(p.ring) + ru, u);
                    else
                        store_cols<CPL>(static_cast<float*>(p.ring) + ru, u);
                }
                if (it.vt == 0 && lane == 0) ring_put(p, rec + K + p.G * V + it.m, a);
                rec += p.ring_tok;
            }
            if constexpr (SNAP) {
                if (--snap_left == 0) {
                    snap_left = p.spt;
                    if (snap_i < p.snap_count) store_tile(snap, kg, scale, S);
                    ++snap_i;
                    snap += p.snap_tok;
                }
            }
        }
    }

    // Both K-reductions of a token in one pass over the registers, their
    // chains interleaved: o = S^T q and x = S^T k, each in the order of
    // dot_rows (so the same bits).
    __device__ static void dot_rows2(const float (&S)[R][CPL], const float (&qv)[R],
                                     const float (&kv)[R], float (&o)[CPL], float (&x)[CPL]) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            o[c] = S[0][c] * qv[0];
            x[c] = S[0][c] * kv[0];
        }
#pragma unroll
        for (int ri = 1; ri < R; ++ri)
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                o[c] = __builtin_fmaf(S[ri][c], qv[ri], o[c]);
                x[c] = __builtin_fmaf(S[ri][c], kv[ri], x[c]);
            }
    }

    // True when no token of the stage can take the running scale out of
    // [2^-64, 2^64], so the tokens may skip decay_step's test: every decay is
    // positive and finite and the exact products scale * a_1 * ... * a_t stay
    // within [2^-62, 2^62] (the float32 products differ from them by far less
    // than a factor of 2).  Lane t holds log2 of token t's decay and the lanes
    // form prefix sums; wave-uniform.
    __device__ static bool stage_in_range(const float* A, int Lc, float scale, int lane) {
        bool bad = false;
        float l = 0.0f;
        if (lane < Lc) {
            const float a = A[lane];
            bad = !(a > 0.0f && a < __builtin_inff());  // zero, negative, inf or NaN
            l = __builtin_amdgcn_logf(a);                // log2
        }
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            if (d >= C) break;
            const float y = __shfl_up(l, d);
            if (lane >= d) l += y;
        }
        const float ls = __builtin_amdgcn_logf(scale);
        const bool ok = lane >= Lc || (!bad && l + ls >= -62.0f && l + ls <= 62.0f);
        return __ballot(!ok) == 0;
    }

    // The tokens of a multi-token stage (the row-groups-low layout of the
    // long-row shapes): as run_chunk, with the next token's retrieval computed
    // unconditionally in the same register pass as this token's read-out
    // (after the stage's last token it reads a k_hat slot that holds no token
    // of the row and the value is discarded), and the decay range test made
    // once per stage when CHECK is false.  x holds the retrieval of the
    // current token, one value per column.
    template <bool CHECK, bool REC, bool SNAP, bool BC>
    __device__ static void stage_tokens(const RecParams& p, const Item& it, int tc, int Lc,
                                        const float* B, float (&S)[R][CPL], float& scale,
                                        float (&kr)[R], float (&x)[CPL], int w, int lane) {
        static_assert(KG_LOW, "stage_tokens serves the row-groups-low layout");
        const int kg = row_group(lane);
        const int vc = col_chunk(lane) * CPL;
        WT* outp = out_ptr(p, it) + static_cast<int64_t>(tc) * p.o_tok;
        int64_t rec = 0;
        if (REC && it.record)
            rec = static_cast<int64_t>(p.ring_idx[it.row]) * p.ring_row +
                  static_cast<int64_t>(it.h) * p.ring_head + static_cast<int64_t>(tc) * p.ring_tok;
        ST* snap = nullptr;
        int snap_left = 0;
        if constexpr (SNAP) {
            snap_left = p.spt - tc % p.spt;
            snap = static_cast<ST*>(p.snap) + static_cast<int64_t>(it.slot) * p.snap_slot +
                   static_cast<int64_t>(tc / p.spt) * p.snap_tok +
                   static_cast<int64_t>(it.hv) * p.snap_head + it.j0;
        }
        int snap_i = SNAP ? tc / p.spt : 0;
        for (int tau = 0; tau < Lc; ++tau) {
            const float a = B[OFF_A + w * C + tau];
            const float b = BC ? 1.0f : B[OFF_B + w * C + tau];
            const float cn = scale * a;
            float u[CPL];
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) {
                const float vv = B[OFF_V + w * VTOT + tau * BV + vc + cc];
                const float be = BC ? B[OFF_BV + w * VTOT + tau * BV + vc + cc] : b;
                u[cc] = be * (vv - cn * x[cc]);
            }
            scale = CHECK ? decay_step<R, CPL>(S, cn) : cn;
            const float rho = __builtin_amdgcn_rcpf(scale);
            float us[CPL];
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) us[cc] = u[cc] * rho;
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc)
#pragma unroll
                for (int ri = 0; ri < R; ++ri) S[ri][cc] = __builtin_fmaf(kr[ri], us[cc], S[ri][cc]);
            float qr[R], o[CPL], xk[CPL];
            read_rows<R>(B + OFF_Q + tau * KP, kg, qr);
            read_rows<R>(B + OFF_K + (tau + 1) * KP, kg, kr);
            dot_rows2(S, qr, kr, o, xk);
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) {
                o[cc] = scale * sum_row_groups<true>(o[cc]);
                x[cc] = sum_row_groups<true>(xk[cc]);
            }
            // every lane holds its columns' totals: the 8 lanes of a column
            // store the same bits to the same address
            store_cols<CPL>(outp, o);
            outp += p.o_tok;
            if (REC && it.record) {
                const int64_t ru = rec + K + it.m * V + it.j0;
                if (kg == 0) {
                    if (p.ring_bf16)
                        store_cols<CPL>(static_cast<uint16_t*>(p.ring) + ru, u);
                    else
                        store_cols<CPL>(static_cast<float*>(p.ring) + ru, u);
                }
                if (it.vt == 0 && lane == 0) ring_put(p, rec + K + p.G * V + it.m, a);
                rec += p.ring_tok;
            }
            if constexpr (SNAP) {
                if (--snap_left == 0) {
                    snap_left = p.spt;
                    if (snap_i < p.snap_count) store_tile(snap, kg, scale, S);
                    ++snap_i;
                    snap += p.snap_tok;
                }
            }
        }
    }

    // A multi-token stage of the row-groups-low layout: the retrieval of its
    // first token, the stage-wide decay range test, then the tokens.
    template <bool REC, bool SNAP, bool BC>
    __device__ static void run_stage(const RecParams& p, const Item& it, int c, const float* B,
                                     float (&S)[R][CPL], float& scale, int w, int lane) {
        static_assert(C > 1 && KG_LOW, "multi-token stages of the row-groups-low layout");
        const int kg = row_group(lane);
        const int tc = c * C;
        const int Lc = __builtin_amdgcn_readfirstlane(min(C, it.L - tc));
        float kr[R], x[CPL];
        read_rows<R>(B + OFF_K, kg, kr);
        float xc[CPL];
        dot_rows<R, CPL>(S, kr, xc);
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) x[cc] = sum_row_groups<true>(xc[cc]);
        if (stage_in_range(B + OFF_A + w * C, Lc, scale, lane))
            stage_tokens<false, REC, SNAP, BC>(p, it, tc, Lc, B, S, scale, kr, x, w, lane);
        else
            stage_tokens<true, REC, SNAP, BC>(p, it, tc, Lc, B, S, scale, kr, x, w, lane);
    }

    // MODE: kPlain (forward, fused update without snapshots), kVerify (rows
    // that fit the ring record it; longer rows run as kPlain), kSnap; with
    // kBetaCols, beta is read per value column.
    template <int MODE>
    __device__ static void run_chunk_mode(const RecParams& p, const Item& it, int c,
                                          const float* B, float (&S)[R][CPL], float& scale, int w,
                                          int lane) {
        // the long-row shapes' tokens interleave two reductions (registers to
        // spare); the short-row shapes' token loop fills the register budget
        // as it is
        if constexpr (KG_LOW && C > 1)
            run_stage<(MODE & 3) == kVerify, (MODE & 3) == kSnap, (MODE & kBetaCols) != 0>(
                p, it, c, B, S, scale, w, lane);
        else
            run_chunk<(MODE & 3) == kVerify, (MODE & 3) == kSnap, (MODE & kBetaCols) != 0>(
                p, it, c, B, S, scale, w, lane);
    }

    // Stage buffers in LDS: two for the short-row shapes (the next stage is
    // committed while other waves still read the current one); one for the
    // long-row shapes, with a second barrier per chunk, so their 32-token
    // stages fit three workgroups per CU.
    static constexpr int kStageBufs = KG_LOW ? 1 : 2;

    // A committed stage becomes readable: a workgroup barrier, or for the
    // one-token stages (each wave reads only what it wrote) the wave's own
    // LDS writes completing before its lanes read each other's values.
    __device__ static void stage_sync() {
        if constexpr (kPrivStage) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        } else {
            __syncthreads();
        }
    }

    // All chunks of an item whose loaded state is rs and whose chunk-0 inputs
    // are in st; leaves the final state as scale * S.  The state is widened
    // after the first stage is committed, so its loads complete under that
    // work.
    template <int MODE>
    __device__ static void run_item(const RecParams& p, const Item& it, const RawState& rs,
                                    float (&S)[R][CPL], float& scale, Stage& st, float* lds,
                                    int w, int lane) {
        constexpr bool BC = (MODE & kBetaCols) != 0;
        constexpr int BUF = buf<BC>();
        commit_stage<BC>(p, it, 0, st, lds, w, lane);
        stage_sync();
        __builtin_amdgcn_sched_barrier(0);  // keep the widening (and its wait) here
        widen_state(rs, S);
        scale = 1.0f;
        const int nch = (it.L + C - 1) / C;
        for (int c = 0; c < nch; ++c) {
            const bool next = c + 1 < nch;
            // The long-row and one-token shapes issue the next stage's loads
            // before this stage's tokens; the short-row shapes after them, so
            // the loaded registers are not held through the token loop (which
            // lets the 4-column shape run 4 waves per SIMD; their rows mostly
            // fit one stage anyway).
            constexpr bool kLateLoads = !KG_LOW && C > 1;
            if (!kLateLoads && next) load_stage<BC>(p, it, c + 1, st, w, lane);
            run_chunk_mode<MODE>(p, it, c, lds + (kStageBufs == 2 ? (c & 1) * BUF : 0), S, scale,
                                 w, lane);
            if (next) {
                if (kLateLoads) load_stage<BC>(p, it, c + 1, st, w, lane);
                if constexpr (kStageBufs == 1) __syncthreads();  // the stage has been read
                commit_stage<BC>(p, it, c + 1, st, lds + (kStageBufs == 2 ? ((c + 1) & 1) * BUF : 0),
                                 w, lane);
                stage_sync();
            }
        }
    }
};

// Row of the given rank when rows are taken longest first (ties by index):
// long rows start early and short ones fill the end of the launch, instead of
// a long row that happens to sit late in the batch starting last.  Every
// workgroup ranks the rows itself from the offsets: each row's length bucket
// and a bucket histogram in LDS, a wave prefix sum over the histogram, then a
// ballot scan for the k-th row of the rank's bucket.  Called by every thread
// of the workgroup (two barriers) with kOrderBuckets + B words of LDS;
// returns a wave-uniform row in [0, B).
// Length buckets: one per length below 32, then four per octave (the two
// bits after the leading one) up to 8191; longer rows share the last.  Bucket
// 0 holds the longest rows.
__device__ inline uint32_t order_bucket(uint32_t len) {
    uint32_t b = len;
    if (len >= 32) {
        const uint32_t e = 31 - __builtin_clz(len);  // floor(log2(len)) >= 5
        b = 32 + 4 * (e - 5) + ((len >> (e - 2)) & 3);
    }
    const uint32_t top = kOrderBuckets - 1;
    return top - (b < top ? b : top);
}

__device__ int ordered_row(const uint32_t* off, int B, int rank, uint32_t* scratch) {
    static_assert(kOrderBuckets == 64, "one bucket per lane");
    uint32_t* hist = scratch;
    uint32_t* bucket_of = scratch + kOrderBuckets;
    const int t = threadIdx.x;
    const int lane = t & 63;
    if (t < kOrderBuckets) hist[t] = 0;
    __syncthreads();
    for (int i = t; i < B; i += blockDim.x) {
        const uint32_t b = order_bucket(off[i + 1] - off[i]);
        bucket_of[i] = b;
        atomicAdd(&hist[b], 1u);
    }
    __syncthreads();
    const uint32_t h = hist[lane];
    uint32_t incl = h;  // inclusive prefix sum over the 64 buckets
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t x = __shfl_up(incl, d);
        if (lane >= d) incl += x;
    }
    const uint32_t r = static_cast<uint32_t>(rank);
    const uint64_t hit = __ballot(incl - h <= r && r < incl);
    if (hit == 0) return rank;  // rank >= B: not reached for a valid launch
    const int bucket = __ffsll(static_cast<unsigned long long>(hit)) - 1;
    int k = static_cast<int>(r - __shfl(incl - h, bucket));
    for (int c = 0; c < B; c += 64) {
        const int i = c + lane;
        const bool m = i < B && static_cast<int>(bucket_of[i]) == bucket;
        const uint64_t mask = __ballot(m);
        const int cnt = __popcll(mask);
        if (k < cnt) {
            const int below = __popcll(mask & ((uint64_t{1} << lane) - 1));
            const uint64_t sel = __ballot(m && below == k);
            return c + __ffsll(static_cast<unsigned long long>(sel)) - 1;
        }
        k -= cnt;
    }
    return rank;
}

// One work item per workgroup.
// Waves per SIMD asked of the register allocator: the one-token (HBM-bound
// decode) stages 4, or 2 at 8 columns per lane; the short-row shapes of at most
// 4 columns at K <= 128 4 (verify window: -3.6%); the long-row shapes at
// K <= 128 3 (their workgroups' LDS allows 3 per CU); the rest as many as fit.
template <int K, int C, int CPL, bool KG_LOW>
constexpr int kMinWaves = C == 1 ? (CPL <= 4 ? 4 : 2)
                        : (K <= 128 && CPL <= 4 ? (KG_LOW ? (CPL == 1 ? 3 : 2) : 4) : 1);

template <int K, int V, int CPL, int C, int WPG, typename ST, bool KG_LOW, typename WT, int MODE>
__global__ void __launch_bounds__(WPG * 64, (kMinWaves<K, C, CPL, KG_LOW>)) rec_kernel(const RecParams p) {
    using Q = Rec<K, V, CPL, C, WPG, ST, KG_LOW, WT>;
    // stage buffers, then (long-row shapes) the row ranking's words
    constexpr int kStageWords = Q::kStageBufs * Q::template buf<(MODE & kBetaCols) != 0>();
    constexpr int kRankWords = C > 1 && KG_LOW ? kOrderBuckets + kOrderMaxRows : 0;
    __shared__ __attribute__((aligned(16))) float lds[kStageWords + kRankWords];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int kg = Q::row_group(lane);
    int idx = blockIdx.x;
    // Workgroups are dispatched to the 8 XCDs round robin (block b to XCD
    // b % 8).  The parts of one (row, key head) read the same q and k, so they
    // are given blocks 8 apart: one XCD, one L2, while consecutive (row, key
    // head) pairs still spread over all XCDs.
    if (p.parts > 1 && (p.rows * p.nk) % 8 == 0) {
        const int q = idx >> 3;
        const int qp = fdiv(q, p.div_parts);
        idx = (qp * 8 + (idx & 7)) * p.parts + (q - qp * p.parts);
    }
    if (C > 1 && p.order) {  // set for multi-token shapes only
        const int per_row = p.parts * p.nk;
        const int rank = fdiv(idx, p.div_row);
        // The short-row shapes rank in their second stage buffer: the first
        // write there (chunk 1's commit) comes after a barrier that every wave
        // reaches only once it has ranked.  The long-row shapes (one stage
        // buffer) rank in words of their own.
        constexpr int BUF = Q::template buf<(MODE & kBetaCols) != 0>();
        static_assert(C == 1 || KG_LOW || BUF >= kOrderBuckets + kOrderMaxRows, "ranking LDS");
        uint32_t* scratch = reinterpret_cast<uint32_t*>(lds + (KG_LOW ? kStageWords : BUF));
        const int row = __builtin_amdgcn_readfirstlane(ordered_row(p.offsets, p.rows, rank, scratch));
        idx = row * per_row + (idx - rank * per_row);
    }
    const Item it = Q::item(p, idx, w, lane);
    if (it.pad) {
        Q::zero_output(p, it, lane);
        return;
    }
    if (it.L <= 0) return;
    // The first stage's loads are issued before the state's, so that both
    // are in flight together.
    typename Q::Stage st;
    Q::template load_stage<(MODE & kBetaCols) != 0>(p, it, 0, st, w, lane);
    typename Q::RawState rs;
    Q::load_state(p, it, kg, rs);
    float S[Q::R][CPL];
    float scale;
    Q::template run_item<MODE>(p, it, rs, S, scale, st, lds, w, lane);
    Q::store_state(p, it, kg, scale, S);
}

}  // namespace

template <int K, int V, int CPL, int C, typename ST, bool KG_LOW, typename WT, int MODE>
static hipError_t launch_rec_mode(const RecParams& p, int wpg, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(p.rows) * p.nk * p.parts);
    constexpr int TILES = V / (kLanesPerRow * CPL);
    if constexpr (TILES % 4 == 0) {  // every head splits into a multiple of 4 waves
        if (wpg != 4) return hipErrorInvalidValue;
        hipLaunchKernelGGL((rec_kernel<K, V, CPL, C, 4, ST, KG_LOW, WT, MODE>), grid, dim3(256), 0, stream, p);
    } else {
        switch (wpg) {
            case 1: hipLaunchKernelGGL((rec_kernel<K, V, CPL, C, 1, ST, KG_LOW, WT, MODE>), grid, dim3(64), 0, stream, p); break;
            case 2: hipLaunchKernelGGL((rec_kernel<K, V, CPL, C, 2, ST, KG_LOW, WT, MODE>), grid, dim3(128), 0, stream, p); break;
            case 4: hipLaunchKernelGGL((rec_kernel<K, V, CPL, C, 4, ST, KG_LOW, WT, MODE>), grid, dim3(256), 0, stream, p); break;
            default: return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

// One (work type, state type, mode) table of recurrence launch shapes.  Each
// table is instantiated in a translation unit of its own (gdr_rec_table.hip),
// so the library compiles in parallel.
template <typename WT, typename ST, int MODE>
hipError_t launch_rec_table(const RecParams& p, const LaunchShape& s, hipStream_t stream) {
#define GDR_REC_CASE(KK, VV, CC, CH, KL)                                              \
    if (s.K == KK && s.V == VV && s.cpl == CC && s.chunk == CH && s.kg_low == KL)    \
        return launch_rec_mode<KK, VV, CC, CH, ST, KL, WT, MODE>(p, s.wpg, stream);
    GDR_REC_CASE(128, 128, kDecodeCpl, kDecodeChunk, kDecodeKgLow)
    GDR_REC_CASE(128, 128, kTinyCpl, kDecodeChunk, kDecodeKgLow)
    GDR_REC_CASE(128, 128, kShortCpl, kShortChunk, kShortKgLow)
    GDR_REC_CASE(128, 128, kFusedCpl, kFusedChunk, kFusedKgLow)
    GDR_REC_CASE(128, 128, kLongCpl, kLongChunk, kLongKgLow)
    GDR_REC_CASE(256, 256, 2, 8, false)
    GDR_REC_CASE(256, 256, 1, 8, true)
    GDR_REC_CASE(64, 64, 8, 8, false)
    GDR_REC_CASE(64, 64, 2, 16, true)
    GDR_REC_CASE(32, 32, 4, 8, false)
    GDR_REC_CASE(32, 32, 2, 16, true)
    GDR_REC_CASE(16, 16, 2, 8, false)
    GDR_REC_CASE(16, 16, 2, 16, true)
    if constexpr ((MODE & 3) != kVerify) {  // K != V: the fused update only
        GDR_REC_CASE(64, 128, 8, 8, false)
        GDR_REC_CASE(64, 128, 2, 16, true)
        GDR_REC_CASE(128, 64, 1, 16, true)
        GDR_REC_CASE(128, 256, kFusedCpl, kFusedChunk, kFusedKgLow)
        GDR_REC_CASE(128, 64, kFusedCpl, kFusedChunk, kFusedKgLow)
        GDR_REC_CASE(128, 256, 1, 16, true)
        GDR_REC_CASE(256, 128, 2, 8, false)
        GDR_REC_CASE(256, 128, 1, 8, true)
    }
#undef GDR_REC_CASE
    return hipErrorInvalidValue;
}

}  // namespace gdr
