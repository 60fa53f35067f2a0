// Wavefront top-k of one token's router logits (device code, header-only so
// that every router kernel shares it).
//
// ONNX export card, "Truthful graph contracts", row "Router": softmax in fp32,
// top-k, renormalise, per-expert scale. The selection takes K rounds of a
// wavefront maximum over order-preserving 32-bit keys of the fp32 logits (no
// LDS round trips: reductions through DPP, the lowest index among equal keys
// through ballots).
#pragma once
#include "common.h"

namespace moe {

constexpr int kMaxTopK = 8;
constexpr int kMaxExperts = 256;

// fp32 -> unsigned key with the same order (equal floats, including -0 and
// +0, get equal keys; NaN sorts below everything)
__device__ __forceinline__ uint32_t order_key(float f) {
    if (f != f) return 0u;
    const uint32_t u = f == 0.f ? 0u : __float_as_uint(f);  // -0 ties with +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Wavefront-wide reductions through DPP row shifts and row broadcasts (no
// LDS): within each 16-lane row the running value moves up by 1, 2, 4, 8 lanes,
// so lane 15 of a row holds the row's result; row_bcast:15 and row_bcast:31
// then fold the rows so that lane 63 holds the wavefront's. Lanes a shift
// reads from outside the row contribute the identity.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xf, false);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp_u32<0x111, 0xf>(v));  // row_shr:1
    v = max(v, dpp_u32<0x112, 0xf>(v));  // row_shr:2
    v = max(v, dpp_u32<0x114, 0xf>(v));  // row_shr:4
    v = max(v, dpp_u32<0x118, 0xf>(v));  // row_shr:8
    v = max(v, dpp_u32<0x142, 0xa>(v));  // row_bcast:15 into rows 1, 3
    v = max(v, dpp_u32<0x143, 0xc>(v));  // row_bcast:31 into rows 2, 3
    return __builtin_amdgcn_readlane(v, 63);
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add_f32(float x) {
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf, false));
}
__device__ __forceinline__ float wave_sum_f32(float v) {
    v = dpp_add_f32<0x111, 0xf>(v);
    v = dpp_add_f32<0x112, 0xf>(v);
    v = dpp_add_f32<0x114, 0xf>(v);
    v = dpp_add_f32<0x118, 0xf>(v);
    v = dpp_add_f32<0x142, 0xa>(v);
    v = dpp_add_f32<0x143, 0xc>(v);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// inverse of order_key (key 0, a NaN, maps back to a NaN)
__device__ __forceinline__ float key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Run by a full wavefront. lv[j]: the token's logit of expert lane + 64 j
// (E <= 256; entries with that index >= E are ignored).
// softmax over all E in fp32 (max-subtracted), then the top K by logit; the K
// probabilities are renormalised to sum 1 (summed in k order) and multiplied
// by the per-expert scale. Every lane ends with the same ik[0..K), wk[0..K).
// Selection: K rounds; each takes the largest remaining key (a wavefront
// maximum) and, among equal keys, the lowest expert index (ballots in index
// order), so the experts come out in descending logit, ties to the lower index.
// pv (used when PV): pv[j] = pes[lane + 64 j] already in registers, so that no
// load waits on the selection.
template <bool PV = false>
__device__ __forceinline__ void wave_topk_vals(const float (&lv)[4], const float* __restrict__ pes,
                                               int E, int K, int lane, int* ik, float* wk,
                                               const float (&pv)[4] = {0.f, 0.f, 0.f, 0.f}) {
    uint32_t key[4];
    bool avail[4];
    const int nj = (E + kWave - 1) / kWave;  // uniform
    uint32_t kmax = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        avail[j] = j < nj && lane + kWave * j < E;
        key[j] = avail[j] ? order_key(lv[j]) : 0u;
        kmax = max(kmax, key[j]);
    }
    const float m = key_value(wave_max_u32(kmax));
    float ex[4], sl = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        ex[j] = avail[j] ? expf(lv[j] - m) : 0.f;
        sl += ex[j];
    }
    const float s = wave_sum_f32(sl);

    float pk[kMaxTopK], sk[kMaxTopK];
    float psum = 0.f;
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) {
        ik[k] = 0;
        pk[k] = 0.f;
        sk[k] = 0.f;
        if (k < K) {  // uniform
            uint32_t local = 0u;
#pragma unroll
            for (int j = 0; j < 4; ++j) local = max(local, avail[j] ? key[j] : 0u);
            const uint32_t M = wave_max_u32(local);
            int sj = -1, sl_ = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (j < nj && sj < 0) {
                    const unsigned long long b = __ballot(avail[j] && key[j] == M);
                    if (b) {
                        sj = j;
                        sl_ = __ffsll((long long)b) - 1;
                    }
                }
            }
            // sj >= 0: at least K <= E experts are available
            float e_sel = ex[0], p_sel = pv[0];
#pragma unroll
            for (int j = 1; j < 4; ++j)
                if (sj == j) {
                    e_sel = ex[j];
                    p_sel = pv[j];
                }
            ik[k] = sl_ + kWave * sj;
            pk[k] = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(e_sel), sl_)) / s;
            if (PV) sk[k] = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(p_sel), sl_));
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (sj == j && lane == sl_) avail[j] = false;
            psum += pk[k];
        }
    }
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) wk[k] = (k < K) ? pk[k] / psum * (PV ? sk[k] : pes[ik[k]]) : 0.f;
}

// Same, with the logits read from lrow[0..E).
__device__ __forceinline__ void wave_topk(const float* __restrict__ lrow,
                                          const float* __restrict__ pes, int E, int K, int lane,
                                          int* ik, float* wk) {
    float lv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = lane + kWave * j;
        lv[j] = e < E ? lrow[e] : 0.f;
    }
    wave_topk_vals(lv, pes, E, K, lane, ik, wk);
}

}  // namespace moe
