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
// reads from outside the row contribute OLD, the identity of the reduction.
template <int CTRL, int ROW_MASK, uint32_t OLD>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)OLD, (int)v, CTRL, ROW_MASK, 0xf, false);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp_u32<0x111, 0xf, 0u>(v));  // row_shr:1
    v = max(v, dpp_u32<0x112, 0xf, 0u>(v));  // row_shr:2
    v = max(v, dpp_u32<0x114, 0xf, 0u>(v));  // row_shr:4
    v = max(v, dpp_u32<0x118, 0xf, 0u>(v));  // row_shr:8
    v = max(v, dpp_u32<0x142, 0xa, 0u>(v));  // row_bcast:15 into rows 1, 3
    v = max(v, dpp_u32<0x143, 0xc, 0u>(v));  // row_bcast:31 into rows 2, 3
    return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    v = min(v, dpp_u32<0x111, 0xf, 0xFFFFFFFFu>(v));
    v = min(v, dpp_u32<0x112, 0xf, 0xFFFFFFFFu>(v));
    v = min(v, dpp_u32<0x114, 0xf, 0xFFFFFFFFu>(v));
    v = min(v, dpp_u32<0x118, 0xf, 0xFFFFFFFFu>(v));
    v = min(v, dpp_u32<0x142, 0xa, 0xFFFFFFFFu>(v));
    v = min(v, dpp_u32<0x143, 0xc, 0xFFFFFFFFu>(v));
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
// The top K by logit, then their renormalised softmax weights times the
// per-expert scale. Every lane ends with the same ik[0..K), wk[0..K).
// Selection: K rounds, without branches; each takes the largest remaining key
// (a wavefront maximum of order_key + 1; 0 marks a taken or absent expert)
// and, among equal keys, the lowest expert index (a wavefront minimum of the
// indices holding it), so the experts come out in descending logit, ties to
// the lower index. Weights: exp(l_k - l_0) / sum_j exp(l_j - l_0) over the K
// selected (summed in k order), which is the softmax over all E renormalised
// over the selection: the full denominator cancels.
// pv (used when PV): pv[j] = pes[lane + 64 j] already in registers, so that no
// load waits on the selection.
template <bool PV = false>
__device__ __forceinline__ void wave_topk_vals(const float (&lv)[4], const float* __restrict__ pes,
                                               int E, int K, int lane, int* ik, float* wk,
                                               const float (&pv)[4] = {0.f, 0.f, 0.f, 0.f}) {
    uint32_t key[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) key[j] = (lane + kWave * j < E) ? order_key(lv[j]) + 1u : 0u;
    float lk[kMaxTopK], sk[kMaxTopK];
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) {
        ik[k] = 0;
        lk[k] = 0.f;
        sk[k] = 0.f;
        if (k < K) {  // uniform
            const uint32_t M = wave_max_u32(max(max(key[0], key[1]), max(key[2], key[3])));
            uint32_t ci = 0xFFFFFFFFu;
#pragma unroll
            for (int j = 3; j >= 0; --j)
                if (key[j] == M) ci = (uint32_t)(lane + kWave * j);
            const uint32_t sel = wave_min_u32(ci);  // M > 0 while K <= E
            const int jsel = (int)(sel >> 6), lsel = (int)(sel & 63);
            ik[k] = (int)sel;
            lk[k] = key_value(M - 1u);
            if (PV) {
                const float p = jsel == 0 ? pv[0] : jsel == 1 ? pv[1] : jsel == 2 ? pv[2] : pv[3];
                sk[k] = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(p), lsel));
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if ((uint32_t)(lane + kWave * j) == sel) key[j] = 0u;
        }
    }
    float ex[kMaxTopK], sum = 0.f;
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) {
        ex[k] = k < K ? expf(lk[k] - lk[0]) : 0.f;
        sum += ex[k];
    }
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) wk[k] = (k < K) ? ex[k] / sum * (PV ? sk[k] : pes[ik[k]]) : 0.f;
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
