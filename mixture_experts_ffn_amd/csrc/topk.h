// Wavefront top-k of one token's router logits (device code, header-only so
// that the router and the fused small-batch grouping kernel share it).
#pragma once
#include "common.h"

namespace moe {

constexpr int kMaxTopK = 8;
constexpr int kMaxExperts = 256;

// Run by a full wavefront. lrow: the token's E fp32 logits (E <= 256).
// softmax over all E in fp32 (max-subtracted), then K rounds of a wavefront
// argmax: larger logit wins, equal logits go to the lower expert index.
// The K selected probabilities are renormalised to sum 1 (summed in k order)
// and multiplied by the per-expert scale. Every lane ends with the same
// ik[0..K) and wk[0..K).
__device__ __forceinline__ void wave_topk(const float* __restrict__ lrow,
                                          const float* __restrict__ pes, int E, int K, int lane,
                                          int* ik, float* wk) {
    float l[4], ex[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = lane + kWave * j;
        l[j] = (e < E) ? lrow[e] : -INFINITY;
    }
    float m = fmaxf(fmaxf(l[0], l[1]), fmaxf(l[2], l[3]));
    m = wave_max<kWave>(m);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = lane + kWave * j;
        ex[j] = (e < E) ? expf(l[j] - m) : 0.f;
        s += ex[j];
    }
    s = wave_sum<kWave>(s);

    unsigned sel = 0u;
    float pk[kMaxTopK];
    float psum = 0.f;
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) {
        ik[k] = 0;
        pk[k] = 0.f;
        if (k < K) {
            float bv = -INFINITY, bp = 0.f;
            int bi = 0x7fffffff;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int e = lane + kWave * j;
                // ascending j is ascending e: a strict '>' keeps the lower index on ties.
                // The first unselected expert is always taken, so a NaN or -inf
                // logit can never leave the winner unset (bi stays a valid index).
                if (e < E && !((sel >> j) & 1u) && (bi == 0x7fffffff || l[j] > bv)) {
                    bv = l[j];
                    bi = e;
                    bp = ex[j];
                }
            }
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
                const float ov = __shfl_xor(bv, off, kWave);
                const int oi = __shfl_xor(bi, off, kWave);
                const float op = __shfl_xor(bp, off, kWave);
                if (ov > bv || (ov == bv && oi < bi)) {
                    bv = ov;
                    bi = oi;
                    bp = op;
                }
            }
            if ((bi & (kWave - 1)) == lane) sel |= 1u << (bi >> 6);
            ik[k] = bi;
            pk[k] = bp / s;
            psum += pk[k];
        }
    }
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) wk[k] = (k < K) ? pk[k] / psum * pes[ik[k]] : 0.f;
}

}  // namespace moe
