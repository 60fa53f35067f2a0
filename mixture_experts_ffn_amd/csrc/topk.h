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

// Inclusive prefix sum over the wavefront's lanes (lane l gets v_0 + .. +
// v_l): within each 16-lane row by row shifts of 1, 2, 4, 8 (lanes shifted in
// from outside the row add 0), then row 15's total into rows 1 and 3 and lane
// 31's running total into rows 2 and 3.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_add_u32(uint32_t x) {
    return x + (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xf, false);
}
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
    v = dpp_add_u32<0x111, 0xf>(v);
    v = dpp_add_u32<0x112, 0xf>(v);
    v = dpp_add_u32<0x114, 0xf>(v);
    v = dpp_add_u32<0x118, 0xf>(v);
    v = dpp_add_u32<0x142, 0xa>(v);
    v = dpp_add_u32<0x143, 0xc>(v);
    return v;
}

// inverse of order_key (key 0, a NaN, maps back to a NaN)
__device__ __forceinline__ float key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Run by a full wavefront. lv[j]: the token's logit of expert lane + 64 j
// (E <= 64 NJ; entries with that index >= E are ignored).
// The top K by logit, then their renormalised softmax weights times the
// per-expert scale. Every lane ends with the same ik[0..K), wk[0..K).
// Selection: K rounds, without branches; each takes the largest remaining key
// (a wavefront maximum of order_key + 1; 0 marks a taken or absent expert)
// and, among equal keys, the lowest expert index: the lowest j whose ballot of
// key[j] == max is not empty, then the lowest lane in that ballot (expert
// lane + 64 j). So the experts come out in descending logit, ties to the lower
// index. Weights: exp(l_k - l_0) / sum_j exp(l_j - l_0) over the K selected
// (summed in k order), which is the softmax over all E renormalised over the
// selection: the full denominator cancels.
// pv (used when PV): pv[j] = pes[lane + 64 j] already in registers, so that no
// load waits on the selection.
template <bool PV = false, int NJ = 4>
__device__ __forceinline__ void wave_topk_vals(const float (&lv)[4], const float* __restrict__ pes,
                                               int E, int K, int lane, int* ik, float* wk,
                                               const float (&pv)[4] = {0.f, 0.f, 0.f, 0.f}) {
    static_assert(NJ >= 1 && NJ <= 4, "at most 256 experts");
    uint32_t key[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) key[j] = (lane + kWave * j < E) ? order_key(lv[j]) + 1u : 0u;
    float lk[kMaxTopK], sk[kMaxTopK];
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) {
        ik[k] = 0;
        lk[k] = 0.f;
        sk[k] = 0.f;
        if (k < K) {  // uniform
            uint32_t m = key[0];
#pragma unroll
            for (int j = 1; j < NJ; ++j) m = max(m, key[j]);
            const uint32_t M = wave_max_u32(m);  // > 0 while K <= E
            unsigned long long bj[NJ];
#pragma unroll
            for (int j = 0; j < NJ; ++j) bj[j] = __ballot(key[j] == M);
            int jsel = NJ - 1;
            unsigned long long bs = bj[NJ - 1];
#pragma unroll
            for (int j = NJ - 2; j >= 0; --j)
                if (bj[j] != 0ull) {
                    jsel = j;
                    bs = bj[j];
                }
            const int lsel = __ffsll((long long)bs) - 1;
            ik[k] = lsel + kWave * jsel;
            lk[k] = key_value(M - 1u);
            if (PV) {
                float p = pv[0];
#pragma unroll
                for (int j = 1; j < NJ; ++j)
                    if (jsel == j) p = pv[j];
                sk[k] = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(p), lsel));
            }
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                if (j == jsel && lane == lsel) key[j] = 0u;
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
