// gfx950 (CDNA4) kernels of the gated delta rule recurrence.
//
// Method (pages "gated_delta_recurrence_fwd_gpu", summary; and
// "core.ssm.ops.gdp.fused_recurrent", fused_recurrent_gated_delta_rule_fwd_kernel):
// per (sequence, value head) a K x V float32 state is carried token by token:
//     S <- a S;  u = beta (v - S^T k_hat);  S <- S + k_hat u^T;  o = scale S^T q_hat
//
// Work decomposition (ours, for 64-wide waves):
//   * one wave owns the full K extent of BV = 8*CPL contiguous value columns of
//     one value head: lane = 8*kg + vl holds key rows [kg*R, kg*R + R) (R = K/8)
//     of columns [j0, j0 + CPL).  The state stays in VGPRs for the whole row.
//   * the K-reduction of every column (S^T k_hat and S^T q_hat) is an in-lane
//     fused multiply-add chain over the R rows in ascending order followed by
//     an xor butterfly over the 8 lane groups (DPP row_ror:8, then gfx950's
//     v_permlane16_swap / v_permlane32_swap).  This order depends on K only,
//     never on CPL, the chunk size or the workgroup shape, so every launch
//     shape, the verify kernel and the fold produce identical bits.
//   * a workgroup is WPG waves of one (row, key head); q/k of a chunk of C
//     tokens are normalised once per workgroup and staged in LDS together with
//     the chunk's v, decay and beta; the next chunk's global loads are issued
//     before the current chunk is processed.
//   * S^T k_hat of token t+1 is computed in the same register pass as the
//     read-out S^T q_hat of token t, so only one pass over the state is made
//     per token; decay is applied as r = a * (S^T k_hat) on the reduced value.
//   * no MFMA: the token-serial recurrence is not a dense contraction.
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

// Sum over the 8 key-row groups (lanes l, l^8, ..., l^56).
__device__ __forceinline__ float sum_row_groups(float x) {
    x = x + dpp<0x128>(x);  // row_ror:8 is lane ^ 8 inside a 16-lane row
    x = xor16_sum(x);
    x = xor32_sum(x);
    return x;
}

// Sum over the whole wave, identical in every lane.
__device__ __forceinline__ float sum_wave(float x) {
    x = x + dpp<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
    x = x + dpp<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
    x = x + dpp<0x141>(x);  // row_half_mirror: quads are uniform, pairs quad 0/1
    x = x + dpp<0x140>(x);  // row_mirror: half-rows are uniform, pairs them
    x = xor16_sum(x);
    x = xor32_sum(x);
    return x;
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

// ---------------------------------------------------- per-lane arithmetic ---

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

// The R rows [kg*R, kg*R + R) of a K-vector staged in LDS with 4 floats of
// padding after every R (so the 8 row groups hit different banks).
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

template <int R>
__device__ __forceinline__ int pad_index(int i) { return i + (i / R) * 4; }

// ------------------------------------------------------------- recurrence ---

template <int K, int CPL, int C, int WPG, typename ST>
__global__ void __launch_bounds__(WPG * 64) rec_kernel(const RecParams p) {
    constexpr int V = K;
    constexpr int R = K / kRowGroups;
    constexpr int BV = kLanesPerRow * CPL;
    constexpr int TILES = V / BV;
    constexpr int KP = K + 4 * kRowGroups;       // padded staged vector
    constexpr int QK = (K + 63) / 64;            // q/k elements per lane (norm)
    constexpr int SPW = (C + WPG - 1) / WPG;     // tokens normalised per wave
    constexpr int VTOT = C * BV;                 // v floats per wave per chunk
    constexpr int VPL = VTOT >= 64 ? VTOT / 64 : 1;
    static_assert(R >= 2 && TILES >= 1 && V % BV == 0, "tile shape");
    static_assert(VTOT < 64 || VTOT % 64 == 0, "v staging");
    static_assert(C <= 64, "gate staging uses one lane per token");

    constexpr int OFF_K = 0;
    constexpr int OFF_Q = C * KP;
    constexpr int OFF_V = 2 * C * KP;
    constexpr int OFF_A = OFF_V + WPG * VTOT;
    constexpr int OFF_B = OFF_A + WPG * C;
    constexpr int BUF = (OFF_B + WPG * C + 3) / 4 * 4;
    __shared__ __attribute__((aligned(16))) float lds[2 * BUF];

    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int kg = lane >> 3;
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

    int L;
    int64_t rq, rk, rv, rg, rb, ro;
    if (p.offsets) {
        const int64_t t0 = p.offsets[row];
        L = static_cast<int>(static_cast<int64_t>(p.offsets[row + 1]) - t0);
        rq = t0 * p.q_tok; rk = t0 * p.k_tok; rv = t0 * p.v_tok;
        rg = t0 * p.g_tok; rb = t0 * p.b_tok; ro = t0 * p.o_tok;
    } else {
        L = p.dense_len;
        rq = row * p.q_seq; rk = row * p.k_seq; rv = row * p.v_seq;
        rg = row * p.g_seq; rb = row * p.b_seq; ro = row * p.o_seq;
    }
    const uint32_t slot = p.slot_idx ? p.slot_idx[row] : static_cast<uint32_t>(row);
    float* outp = p.out + ro + static_cast<int64_t>(hv) * p.o_head + j0;

    if (p.slot_idx && slot == kPadSlot) {  // padding request: zero output only
        if (kg == 0) {
            float z[CPL];
#pragma unroll
            for (int c = 0; c < CPL; ++c) z[c] = 0.0f;
            for (int t = 0; t < L; ++t) store_cols<CPL>(outp + t * p.o_tok, z);
        }
        return;
    }
    if (L <= 0) return;

    // ---- state tile into registers (issued first: the longest latency) ----
    float S[R][CPL];
    const int64_t src_sel = p.src_by_slot ? static_cast<int64_t>(slot) : row;
    if (p.src) {
        const ST* sp = static_cast<const ST*>(p.src) + src_sel * p.src_slot +
                       static_cast<int64_t>(hv) * p.src_head + j0;
#pragma unroll
        for (int ri = 0; ri < R; ++ri) load_cols<CPL>(sp + (kg * R + ri) * V, S[ri]);
    } else {
#pragma unroll
        for (int ri = 0; ri < R; ++ri)
#pragma unroll
            for (int c = 0; c < CPL; ++c) S[ri][c] = 0.0f;
    }

    const bool record = p.ring != nullptr && L <= p.ring_len;
    float* rec = record ? p.ring + static_cast<int64_t>(p.ring_idx[row]) * p.ring_row +
                              static_cast<int64_t>(h) * p.ring_head
                        : nullptr;

    // ---- chunk staging: global -> registers -> (norms) -> LDS ----
    float sq[SPW][QK], sk[SPW][QK], sv[VPL], sa, sb;

    auto load_stage = [&](int c) {
        const int tc = c * C;
#pragma unroll
        for (int s = 0; s < SPW; ++s) {
            const int tau = w + s * WPG;
            const int t = tc + tau;
            const bool ok = tau < C && t < L;
#pragma unroll
            for (int e = 0; e < QK; ++e) {
                const int idx = lane + 64 * e;
                const bool in = ok && idx < K;
                sq[s][e] = in ? p.q[rq + t * p.q_tok + h * p.q_head + idx] : 0.0f;
                sk[s][e] = in ? p.k[rk + t * p.k_tok + h * p.k_head + idx] : 0.0f;
            }
        }
        {
            const int flat = lane * VPL;
            const int tau = flat / BV;
            const int col = flat - tau * BV;
            const int t = tc + tau;
            const bool ok = flat < VTOT && t < L;
            const float* vp = p.v + rv + t * p.v_tok + hv * p.v_head + vt * BV + col;
            if constexpr (VPL == 4) {
                float4 x = ok ? *reinterpret_cast<const float4*>(vp) : make_float4(0, 0, 0, 0);
                sv[0] = x.x; sv[1] = x.y; sv[2] = x.z; sv[3] = x.w;
            } else if constexpr (VPL == 2) {
                float2 x = ok ? *reinterpret_cast<const float2*>(vp) : make_float2(0, 0);
                sv[0] = x.x; sv[1] = x.y;
            } else {
#pragma unroll
                for (int i = 0; i < VPL; ++i) sv[i] = ok ? vp[i] : 0.0f;
            }
        }
        {
            const int t = tc + lane;
            const bool ok = lane < C && t < L;
            sa = 1.0f;
            sb = 1.0f;
            if (ok && p.gate) {
                const float g = p.gate[rg + t * p.g_tok + hv * p.g_head];
                sa = p.gate_is_log ? expf(g) : g;
            }
            if (ok && p.beta) sb = p.beta[rb + t * p.b_tok + hv * p.b_head];
        }
    };

    auto commit_stage = [&](int c, float* B) {
        const int tc = c * C;
#pragma unroll
        for (int s = 0; s < SPW; ++s) {
            const int tau = w + s * WPG;
            if (tau >= C) break;
            float rk = 1.0f, rqs = p.scale;
            if (p.l2norm) {
                float kk = sk[s][0] * sk[s][0];
                float qq = sq[s][0] * sq[s][0];
#pragma unroll
                for (int e = 1; e < QK; ++e) {
                    kk = __builtin_fmaf(sk[s][e], sk[s][e], kk);
                    qq = __builtin_fmaf(sq[s][e], sq[s][e], qq);
                }
                kk = sum_wave(kk);
                qq = sum_wave(qq);
                rk = rsqrtf(kk + kEps);
                rqs = rsqrtf(qq + kEps) * p.scale;
            }
            const bool rec_k = record && part == 0 && tc + tau < L;
#pragma unroll
            for (int e = 0; e < QK; ++e) {
                const int idx = lane + 64 * e;
                if (idx < K) {
                    const float kh = sk[s][e] * rk;
                    B[OFF_K + tau * KP + pad_index<R>(idx)] = kh;
                    B[OFF_Q + tau * KP + pad_index<R>(idx)] = sq[s][e] * rqs;
                    if (rec_k) rec[(tc + tau) * p.ring_tok + idx] = kh;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int flat = lane * VPL + i;
            if (flat < VTOT) B[OFF_V + w * VTOT + flat] = sv[i];
        }
        if (lane < C) {
            B[OFF_A + w * C + lane] = sa;
            B[OFF_B + w * C + lane] = sb;
        }
    };

    load_stage(0);
    commit_stage(0, lds);
    __syncthreads();

    const int nch = (L + C - 1) / C;
    for (int c = 0; c < nch; ++c) {
        const float* B = lds + (c & 1) * BUF;
        const int tc = c * C;
        const int Lc = min(C, L - tc);
        if (c + 1 < nch) load_stage(c + 1);

        float kr[R];
        read_rows<R>(B + OFF_K, kg, kr);
        float x[CPL];
        dot_rows<R, CPL>(S, kr, x);
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) x[cc] = sum_row_groups(x[cc]);

        for (int tau = 0; tau < Lc; ++tau) {
            const float a = B[OFF_A + w * C + tau];
            const float be = B[OFF_B + w * C + tau];
            float vv[CPL];
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) vv[cc] = B[OFF_V + w * VTOT + tau * BV + vl * CPL + cc];
            float u[CPL];
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) u[cc] = be * (vv[cc] - a * x[cc]);
#pragma unroll
            for (int ri = 0; ri < R; ++ri)
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc)
                    S[ri][cc] = __builtin_fmaf(kr[ri], u[cc], a * S[ri][cc]);

            float qr[R];
            read_rows<R>(B + OFF_Q + tau * KP, kg, qr);
            float o[CPL];
            dot_rows<R, CPL>(S, qr, o);
            const bool more = tau + 1 < Lc;
            if (more) {
                read_rows<R>(B + OFF_K + (tau + 1) * KP, kg, kr);
                dot_rows<R, CPL>(S, kr, x);
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc) x[cc] = sum_row_groups(x[cc]);
            }
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) o[cc] = sum_row_groups(o[cc]);

            const int t = tc + tau;
            if (kg == 0) store_cols<CPL>(outp + t * p.o_tok, o);
            if (record) {
                float* r = rec + t * p.ring_tok;
                if (kg == 0) store_cols<CPL>(r + K + m * V + j0, u);
                if (vt == 0 && lane == 0) r[K + p.G * V + m] = a;
            }
            if (p.snap && (t + 1) % p.spt == 0) {
                const int i = (t + 1) / p.spt - 1;
                if (i < p.snap_count) {
                    ST* sp = static_cast<ST*>(p.snap) + static_cast<int64_t>(slot) * p.snap_slot +
                             static_cast<int64_t>(i) * p.snap_tok +
                             static_cast<int64_t>(hv) * p.snap_head + j0;
#pragma unroll
                    for (int ri = 0; ri < R; ++ri) store_cols<CPL>(sp + (kg * R + ri) * V, S[ri]);
                }
            }
        }
        if (c + 1 < nch) {
            commit_stage(c + 1, lds + ((c + 1) & 1) * BUF);
            __syncthreads();
        }
    }

    if (p.dst && !record) {
        const int64_t dsel = p.dst_by_slot ? static_cast<int64_t>(slot) : row;
        ST* dp = static_cast<ST*>(p.dst) + dsel * p.dst_slot +
                 static_cast<int64_t>(hv) * p.dst_head + j0;
#pragma unroll
        for (int ri = 0; ri < R; ++ri) store_cols<CPL>(dp + (kg * R + ri) * V, S[ri]);
    }
}

// ------------------------------------------------------------------- fold ---

template <int K, int CPL, int WPG, typename ST>
__global__ void __launch_bounds__(WPG * 64) fold_kernel(const FoldParams p) {
    constexpr int V = K;
    constexpr int R = K / kRowGroups;
    constexpr int BV = kLanesPerRow * CPL;
    constexpr int TILES = V / BV;

    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int kg = lane >> 3;
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
    for (int ri = 0; ri < R; ++ri) load_cols<CPL>(sp + (kg * R + ri) * V, S[ri]);

    const float* rec = p.ring + static_cast<int64_t>(p.ring_idx[row]) * p.ring_row +
                       static_cast<int64_t>(h) * p.ring_head;
    for (uint32_t t = 0; t < n; ++t) {
        const float* r = rec + static_cast<int64_t>(t) * p.ring_tok;
        const float a = r[K + p.G * V + m];
        float kr[R];
        if constexpr (R % 4 == 0) {
#pragma unroll
            for (int i = 0; i < R; i += 4) {
                const float4 x4 = *reinterpret_cast<const float4*>(r + kg * R + i);
                kr[i] = x4.x; kr[i + 1] = x4.y; kr[i + 2] = x4.z; kr[i + 3] = x4.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < R; ++i) kr[i] = r[kg * R + i];
        }
        float u[CPL];
        load_cols<CPL>(r + K + m * V + j0, u);
#pragma unroll
        for (int ri = 0; ri < R; ++ri)
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc)
                S[ri][cc] = __builtin_fmaf(kr[ri], u[cc], a * S[ri][cc]);
    }
#pragma unroll
    for (int ri = 0; ri < R; ++ri) store_cols<CPL>(sp + (kg * R + ri) * V, S[ri]);
}

}  // namespace

// ------------------------------------------------------------- dispatch ---

template <int K, int CPL, int C, typename ST>
static hipError_t launch_rec_wpg(const RecParams& p, int wpg, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(p.rows) * p.nk * p.parts);
    switch (wpg) {
        case 1: hipLaunchKernelGGL((rec_kernel<K, CPL, C, 1, ST>), grid, dim3(64), 0, stream, p); break;
        case 2: hipLaunchKernelGGL((rec_kernel<K, CPL, C, 2, ST>), grid, dim3(128), 0, stream, p); break;
        case 4: hipLaunchKernelGGL((rec_kernel<K, CPL, C, 4, ST>), grid, dim3(256), 0, stream, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename ST>
static hipError_t launch_rec_st(const RecParams& p, const LaunchShape& s, hipStream_t stream) {
#define GDR_REC_CASE(KK, CC, CH)                                   \
    if (s.K == KK && s.cpl == CC && s.chunk == CH)                 \
        return launch_rec_wpg<KK, CC, CH, ST>(p, s.wpg, stream);
    GDR_REC_CASE(128, 4, 8)
    GDR_REC_CASE(128, 2, 16)
    GDR_REC_CASE(64, 8, 8)
    GDR_REC_CASE(64, 2, 16)
    GDR_REC_CASE(32, 4, 8)
    GDR_REC_CASE(32, 2, 16)
    GDR_REC_CASE(16, 2, 8)
    GDR_REC_CASE(16, 2, 16)
#undef GDR_REC_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_recurrence(const RecParams& p, const LaunchShape& s, StateType st,
                             hipStream_t stream) {
    return st == StateType::BF16 ? launch_rec_st<uint16_t>(p, s, stream)
                                 : launch_rec_st<float>(p, s, stream);
}

template <int K, int CPL, typename ST>
static hipError_t launch_fold_wpg(const FoldParams& p, int wpg, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(p.rows) * p.nk * p.parts);
    switch (wpg) {
        case 1: hipLaunchKernelGGL((fold_kernel<K, CPL, 1, ST>), grid, dim3(64), 0, stream, p); break;
        case 2: hipLaunchKernelGGL((fold_kernel<K, CPL, 2, ST>), grid, dim3(128), 0, stream, p); break;
        case 4: hipLaunchKernelGGL((fold_kernel<K, CPL, 4, ST>), grid, dim3(256), 0, stream, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename ST>
static hipError_t launch_fold_st(const FoldParams& p, const LaunchShape& s, hipStream_t stream) {
    switch (s.K) {
        case 128: return s.cpl == 4 ? launch_fold_wpg<128, 4, ST>(p, s.wpg, stream) : hipErrorInvalidValue;
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
