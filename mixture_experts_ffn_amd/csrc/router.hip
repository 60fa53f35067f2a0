// Router of the hybrid MoE FFN block on gfx950.
//
// ONNX export card, "Truthful graph contracts", row "Router": a scale-free
// RMSNorm, a learned per-channel scale times hidden^-0.5, a linear map to one
// logit per expert, a softmax in fp32, top-k, renormalisation, then the
// per-expert scale. Everything here runs in fp32: bf16 inputs are widened
// exactly and nothing is rounded back to bf16 before the selection.
#include "common.h"
#include "kernels.h"
#include "topk.h"

namespace moe {

constexpr int kRouterTokens = 8;    // tokens per block
constexpr int kRouterExperts = 16;  // experts per block (4 per wave)

// logits[t, e] = rms(x_t)^-1 * H^-0.5 * sum_h x[t,h] * s[h] * W[e,h] (+ bias[e])
// The per-token factor rms^-1 * H^-0.5 is applied after the dot product (the
// same value up to fp32 rounding as normalising x first).
__global__ __launch_bounds__(256) void router_logits_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ scale,
    const uint16_t* __restrict__ w, const float* __restrict__ bias, int T, int H, int E,
    float eps, float inv_sqrt_h, float* __restrict__ logits) {
    extern __shared__ uint2 xs[];  // [kRouterTokens][H/4], 4 bf16 per entry
    __shared__ float rn[kRouterTokens];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int t0 = blockIdx.y * kRouterTokens;
    const int nt = min(kRouterTokens, T - t0);
    const int hc4 = H >> 2;

    for (int i = tid; i < kRouterTokens * hc4; i += 256) {
        const int t = i / hc4, c = i - t * hc4;
        uint2 v = make_uint2(0u, 0u);
        if (t < nt) v = reinterpret_cast<const uint2*>(x + (size_t)(t0 + t) * H)[c];
        xs[i] = v;
    }
    __syncthreads();

    // scale-free RMSNorm factor per token (wave w: tokens w, w + 4)
    for (int t = wave; t < kRouterTokens; t += 4) {
        float ss = 0.f;
        for (int c = lane; c < hc4; c += kWave) {
            const uint2 v = xs[t * hc4 + c];
            const float a = bf16_lo(v.x), b = bf16_hi(v.x), d = bf16_lo(v.y), f = bf16_hi(v.y);
            ss += a * a + b * b + d * d + f * f;
        }
        ss = wave_sum<kWave>(ss);
        if (lane == 0) rn[t] = 1.0f / sqrtf(ss / (float)H + eps);
    }
    __syncthreads();

    const int nj = H >> 8;  // 4-element chunks per lane
    const uint2* sr = reinterpret_cast<const uint2*>(scale);
    for (int ei = 0; ei < kRouterExperts / 4; ++ei) {
        const int e = blockIdx.x * kRouterExperts + wave * (kRouterExperts / 4) + ei;
        if (e >= E) break;  // uniform across the wave
        const uint2* wr = reinterpret_cast<const uint2*>(w + (size_t)e * H);
        float acc[kRouterTokens];
#pragma unroll
        for (int t = 0; t < kRouterTokens; ++t) acc[t] = 0.f;
        for (int j = 0; j < nj; ++j) {
            const int c = lane + kWave * j;
            const uint2 wv = wr[c], sv = sr[c];
            const float sw0 = bf16_lo(wv.x) * bf16_lo(sv.x), sw1 = bf16_hi(wv.x) * bf16_hi(sv.x);
            const float sw2 = bf16_lo(wv.y) * bf16_lo(sv.y), sw3 = bf16_hi(wv.y) * bf16_hi(sv.y);
#pragma unroll
            for (int t = 0; t < kRouterTokens; ++t) {
                const uint2 xv = xs[t * hc4 + c];
                acc[t] += bf16_lo(xv.x) * sw0 + bf16_hi(xv.x) * sw1 + bf16_lo(xv.y) * sw2 +
                          bf16_hi(xv.y) * sw3;
            }
        }
#pragma unroll
        for (int t = 0; t < kRouterTokens; ++t) acc[t] = wave_sum<kWave>(acc[t]);
        if (lane == 0) {
            const float b = bias ? bias[e] : 0.f;
#pragma unroll
            for (int t = 0; t < kRouterTokens; ++t)
                if (t < nt) logits[(size_t)(t0 + t) * E + e] = acc[t] * (rn[t] * inv_sqrt_h) + b;
        }
    }
}

// One wavefront per token: softmax, top-k, renormalise, per-expert scale.
__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ logits,
                                                          const float* __restrict__ pes, int T,
                                                          int E, int K, int32_t* __restrict__ idx,
                                                          float* __restrict__ wts) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;
    int ik[kMaxTopK];
    float wk[kMaxTopK];
    wave_topk(logits + (size_t)t * E, pes, E, K, lane, ik, wk);
    if (lane == 0) {
#pragma unroll
        for (int k = 0; k < kMaxTopK; ++k)
            if (k < K) {
                idx[(size_t)t * K + k] = ik[k];
                wts[(size_t)t * K + k] = wk[k];
            }
    }
}

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* scale, const uint16_t* w,
                                const float* bias, int T, int H, int E, float eps, float* logits,
                                hipStream_t stream) {
    dim3 grid((E + kRouterExperts - 1) / kRouterExperts, (T + kRouterTokens - 1) / kRouterTokens);
    const size_t lds = (size_t)kRouterTokens * H * sizeof(uint16_t);
    const float inv_sqrt_h = (float)(1.0 / __builtin_sqrt((double)H));
    hipLaunchKernelGGL(router_logits_kernel, grid, dim3(256), lds, stream, x, scale, w, bias, T, H,
                       E, eps, inv_sqrt_h, logits);
    return hipGetLastError();
}

hipError_t launch_router_topk(const float* logits, const float* pes, int T, int E, int K,
                              int32_t* topk_idx, float* topk_w, hipStream_t stream) {
    hipLaunchKernelGGL(router_topk_kernel, dim3((T + 3) / 4), dim3(256), 0, stream, logits, pes, T,
                       E, K, topk_idx, topk_w);
    return hipGetLastError();
}

}  // namespace moe
