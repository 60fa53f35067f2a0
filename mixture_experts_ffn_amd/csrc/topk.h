// Wavefront top-k of one token's router logits (device code, header-only so
// that every router kernel shares it).
//
// ONNX export card, "Truthful graph contracts", row "Router": softmax in fp32,
// top-k, renormalise, per-expert scale. The selection is a radix select over
// order-preserving 32-bit keys of the fp32 logits using wavefront ballots (no
// LDS round trips): the k-th largest key is found bit by bit from the top,
// equal keys at the boundary go to the lower expert index, and the selected
// experts are then ranked (descending logit, ties -> lower index).
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

// Run by a full wavefront. lv[j]: the token's logit of expert lane + 64 j
// (E <= 256; entries with that index >= E are ignored).
// softmax over all E in fp32 (max-subtracted), then the top K by logit; the K
// probabilities are renormalised to sum 1 (summed in k order) and multiplied
// by the per-expert scale. Every lane ends with the same ik[0..K), wk[0..K).
// pv (used when PV): pv[j] = pes[lane + 64 j] already in registers, so that no
// load waits on the selection.
template <bool PV = false>
__device__ __forceinline__ void wave_topk_vals(const float (&lv)[4], const float* __restrict__ pes,
                                               int E, int K, int lane, int* ik, float* wk,
                                               const float (&pv)[4] = {0.f, 0.f, 0.f, 0.f}) {
    float l[4], ex[4];
    uint32_t key[4];
    bool valid[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = lane + kWave * j;
        valid[j] = e < E;
        l[j] = valid[j] ? lv[j] : -INFINITY;
        key[j] = valid[j] ? order_key(l[j]) : 0u;
    }
    const int nj = (E + kWave - 1) / kWave;  // uniform
    float m = fmaxf(fmaxf(l[0], l[1]), fmaxf(l[2], l[3]));
    m = wave_max<kWave>(m);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        ex[j] = valid[j] ? expf(l[j] - m) : 0.f;
        s += ex[j];
    }
    s = wave_sum<kWave>(s);

    // k-th largest key: the largest v with #{key >= v} >= K
    uint32_t prefix = 0u;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = prefix | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (j < nj) cnt += __popcll(__ballot(valid[j] && key[j] >= cand));
        if (cnt >= K) prefix = cand;
    }
    int ngt = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (j < nj) ngt += __popcll(__ballot(valid[j] && key[j] > prefix));
    // take the K - ngt lowest-index experts whose key equals the boundary key
    const int need = K - ngt;
    const unsigned long long below = (1ull << lane) - 1ull;
    bool sel[4];
    int taken = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        sel[j] = false;
        if (j < nj) {
            const unsigned long long meq = __ballot(valid[j] && key[j] == prefix);
            const int r = taken + __popcll(meq & below);
            sel[j] = valid[j] && (key[j] > prefix || (key[j] == prefix && r < need));
            taken += __popcll(meq);
        }
    }
    // rank of each selected expert among the selected: larger key first, then lower index
    int rank[4] = {0, 0, 0, 0};
#pragma unroll
    for (int j2 = 0; j2 < 4; ++j2) {
        if (j2 >= nj) break;
        unsigned long long ms = __ballot(sel[j2]);
        while (ms) {
            const int ln = __ffsll((long long)ms) - 1;
            ms &= ms - 1ull;
            const uint32_t kk = __builtin_amdgcn_readlane(key[j2], ln);
            const int ee = ln + kWave * j2;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int e = lane + kWave * j;
                if (sel[j] && (kk > key[j] || (kk == key[j] && ee < e))) ++rank[j];
            }
        }
    }
    float pk[kMaxTopK], sk[kMaxTopK];
    float psum = 0.f;
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) {
        ik[k] = 0;
        pk[k] = 0.f;
        sk[k] = 0.f;
        if (k < K) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (j < nj) {
                    const unsigned long long mk = __ballot(sel[j] && rank[j] == k);
                    if (mk) {
                        const int ln = __ffsll((long long)mk) - 1;
                        ik[k] = ln + kWave * j;
                        pk[k] = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(ex[j]), ln)) / s;
                        if (PV) sk[k] = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(pv[j]), ln));
                    }
                }
            }
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
