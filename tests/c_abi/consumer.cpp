// A consumer of libgdr.so with no Python and no torch: plain HIP runtime
// calls, gdr_recurrence_fwd on device buffers described by gdr_tensor, and
// the result checked against the CPU oracle (libgdr_oracle.so, test
// infrastructure) on the same inputs.  Also checks that a bad argument is
// reported with its code and message before anything is enqueued.
// Source of the operation: page "gated_delta_recurrence_fwd_gpu" (summary,
// Args).  Prints one line and exits 0 on success.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "gdr.h"

extern "C" int oracle_recurrence_fwd(int B, int nv, int nk, int K, int V,
                                     const uint32_t* row_offsets, const uint32_t* slot_idx,
                                     const float* qkv, const float* decay, const float* beta,
                                     int state_bf16, void* state, int64_t max_slots,
                                     float* out, float scale, int l2norm);

namespace {

#define CHECK_HIP(x)                                                        \
    do {                                                                    \
        hipError_t e_ = (x);                                                \
        if (e_ != hipSuccess) {                                             \
            std::printf("c-abi consumer: %s failed: %s\n", #x,              \
                        hipGetErrorString(e_));                             \
            return 1;                                                       \
        }                                                                   \
    } while (0)

uint64_t g_seed = 0x9E3779B97F4A7C15ull;
float uniform(float lo, float hi) {  // 64-bit LCG, top 24 bits
    g_seed = g_seed * 6364136223846793005ull + 1442695040888963407ull;
    return lo + (hi - lo) * static_cast<float>(g_seed >> 40) / 16777216.0f;
}

gdr_tensor desc(void* data, int32_t dtype, std::vector<int64_t> shape) {
    gdr_tensor t{};
    t.data = data;
    t.dtype = dtype;
    t.ndim = static_cast<int32_t>(shape.size());
    int64_t stride = 1;
    for (int i = t.ndim - 1; i >= 0; --i) {
        t.shape[i] = shape[i];
        t.stride[i] = stride;
        stride *= shape[i];
    }
    return t;
}

double rel_err(const std::vector<float>& got, const std::vector<float>& ref) {
    double num = 0.0, den = 0.0;
    for (size_t i = 0; i < got.size(); ++i) {
        num = std::fmax(num, std::fabs(static_cast<double>(got[i]) - ref[i]));
        den = std::fmax(den, std::fabs(static_cast<double>(ref[i])));
    }
    return den > 0.0 ? num / den : num;
}

}  // namespace

int main() {
    // A ragged batch with an empty row: 3 rows of 5, 0 and 17 tokens, GQA
    // 2 key heads / 4 value heads, K = V = 128, a float32 pool of 6 slots.
    const int B = 3, nk = 2, nv = 4, K = 128, V = 128, slots = 6;
    const std::vector<uint32_t> off = {0, 5, 5, 22};
    const std::vector<uint32_t> slot = {4, 1, 2};
    const int T = static_cast<int>(off[B]);
    const int conv = 2 * nk * K + nv * V;
    const float scale = 1.0f / std::sqrt(static_cast<float>(K));

    std::vector<float> qkv(static_cast<size_t>(T) * conv), decay(T * nv), beta(T * nv);
    std::vector<float> state(static_cast<size_t>(slots) * nv * K * V);
    for (auto& x : qkv) x = uniform(-1.0f, 1.0f);
    for (auto& x : decay) x = uniform(0.5f, 1.0f);
    for (auto& x : beta) x = uniform(0.0f, 1.0f);
    for (auto& x : state) x = uniform(-0.05f, 0.05f);

    void *d_qkv, *d_decay, *d_beta, *d_state, *d_out, *d_off, *d_slot;
    CHECK_HIP(hipMalloc(&d_qkv, qkv.size() * 4));
    CHECK_HIP(hipMalloc(&d_decay, decay.size() * 4));
    CHECK_HIP(hipMalloc(&d_beta, beta.size() * 4));
    CHECK_HIP(hipMalloc(&d_state, state.size() * 4));
    CHECK_HIP(hipMalloc(&d_out, static_cast<size_t>(T) * nv * V * 4));
    CHECK_HIP(hipMalloc(&d_off, off.size() * 4));
    CHECK_HIP(hipMalloc(&d_slot, slot.size() * 4));
    CHECK_HIP(hipMemcpy(d_qkv, qkv.data(), qkv.size() * 4, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_decay, decay.data(), decay.size() * 4, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_beta, beta.data(), beta.size() * 4, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_state, state.data(), state.size() * 4, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_off, off.data(), off.size() * 4, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_slot, slot.data(), slot.size() * 4, hipMemcpyHostToDevice));

    const gdr_tensor t_out = desc(d_out, GDR_DTYPE_F32, {T, nv * V});
    const gdr_tensor t_state = desc(d_state, GDR_DTYPE_F32, {slots, nv, K, V});
    const gdr_tensor t_slot = desc(d_slot, GDR_DTYPE_U32, {B});
    const gdr_tensor t_qkv = desc(d_qkv, GDR_DTYPE_F32, {T, conv});
    const gdr_tensor t_decay = desc(d_decay, GDR_DTYPE_F32, {T, nv});
    const gdr_tensor t_beta = desc(d_beta, GDR_DTYPE_F32, {T, nv});
    const gdr_tensor t_off = desc(d_off, GDR_DTYPE_U32, {B + 1});

    // An argument error is reported before any launch: 4 value heads are not
    // a multiple of 3 key heads.
    int rc = gdr_recurrence_fwd(nv, 3, &t_out, &t_state, &t_slot, &t_qkv, &t_decay, &t_beta,
                                &t_off, scale, GDR_FLAG_L2NORM_QK, nullptr);
    if (rc != GDR_ERR_INVALID_ARG || std::strlen(gdr_last_error_message()) == 0) {
        std::printf("c-abi consumer: bad head counts gave %d\n", rc);
        return 1;
    }

    rc = gdr_recurrence_fwd(nv, nk, &t_out, &t_state, &t_slot, &t_qkv, &t_decay, &t_beta,
                            &t_off, scale, GDR_FLAG_L2NORM_QK, nullptr);
    if (rc != GDR_OK) {
        std::printf("c-abi consumer: gdr_recurrence_fwd returned %d: %s\n", rc,
                    gdr_last_error_message());
        return 1;
    }
    CHECK_HIP(hipDeviceSynchronize());
    std::vector<float> out(static_cast<size_t>(T) * nv * V), got_state(state.size());
    CHECK_HIP(hipMemcpy(out.data(), d_out, out.size() * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(got_state.data(), d_state, got_state.size() * 4,
                        hipMemcpyDeviceToHost));

    std::vector<float> ref_out(out.size(), 0.0f), ref_state = state;
    if (oracle_recurrence_fwd(B, nv, nk, K, V, off.data(), slot.data(), qkv.data(),
                              decay.data(), beta.data(), 0, ref_state.data(), slots,
                              ref_out.data(), scale, 1) != 0) {
        std::printf("c-abi consumer: oracle failed\n");
        return 1;
    }
    const double e_out = rel_err(out, ref_out), e_state = rel_err(got_state, ref_state);
    // Slots 0, 3 and 5 belong to no row, and slot 1's row is empty: untouched.
    const size_t per_slot = static_cast<size_t>(nv) * K * V;
    bool untouched = true;
    for (int s : {0, 1, 3, 5})
        untouched = untouched && std::memcmp(got_state.data() + s * per_slot,
                                             state.data() + s * per_slot, per_slot * 4) == 0;
    for (void* p : {d_qkv, d_decay, d_beta, d_state, d_out, d_off, d_slot}) CHECK_HIP(hipFree(p));
    std::printf("c-abi consumer: ragged forward (rows 5, 0, 17; nk=2, nv=4, K=V=128) through "
                "libgdr.so %s: rel err out %.2e state %.2e, other slots %s\n", gdr_version(),
                e_out, e_state, untouched ? "untouched" : "CHANGED");
    return e_out <= 2e-3 && e_state <= 2e-3 && untouched ? 0 : 1;
}
