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

// ---------------------------------------------------------------------------
// Router for larger batches on MFMA.
//
// logit[t, e] = rms(x_t)^-1 * H^-0.5 * sum_h x[t,h] * (s[h] * W[e,h]) + bias[e].
// s[h] * W[e,h] is a product of two bf16 values, so it has at most 16
// significant bits: it equals hi + lo exactly, with hi its truncation to bf16
// and lo the (bf16-representable) remainder. x is bf16, so the dot product is
// two bf16 MFMAs (x.hi + x.lo) whose products are exact and whose sums
// accumulate in fp32: the logits keep fp32 accuracy, as the router requires.
//
// router_partial_kernel: a workgroup takes 32 tokens, all experts (waves split
//   them in 16-wide column tiles) and one slice of the hidden dimension; it
//   issues the loads of up to NS K-steps at once (no load waits on another),
//   then splits, stages through LDS and multiplies step by step. The sums of
//   each slice go to partial[slice][t][e], and the slice's sum of squares of
//   each token row (from the x chunks it stages) to ss_partial[slice][t].
// router_finish_kernel: one wavefront per token adds the slices in order (the
//   same order for every run), applies the RMSNorm factor from the slices'
//   sums of squares (x is not read again), the H^-0.5 and the bias, and runs
//   the softmax / top-k.
namespace {

constexpr int kRT = 32;  // tokens per workgroup: two 16-row MFMA tiles
constexpr int kRK = 64;  // K-step
constexpr int kRThreads = 256;

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// 16-byte chunk c of LDS row r at chunk c ^ ((r & 7) ^ ((r >> 3) & 1)): 128-bit
// reads of chunk c of 16 consecutive rows (one cycle's 16 lanes over 64 banks)
// then hit 16 distinct (row parity, chunk) bank groups
__device__ __forceinline__ int rswz(int r, int c) { return r * kRK + ((c ^ ((r & 7) ^ ((r >> 3) & 1))) << 3); }

// NQ: router rows staged per thread per K-step (32 NQ experts per workgroup)
template <int NQ>
struct RStage {
    v4u x;       // one 16-byte chunk of the x tile
    v4u w[NQ];   // NQ 16-byte chunks of router rows
    v4u sc;      // the matching 8 router-scale values
};

template <int NQ>
__device__ __forceinline__ void r_load(RStage<NQ>& st, const uint16_t* xr, const uint16_t* const* wr,
                                       const uint16_t* sr, int k0) {
    st.x = *reinterpret_cast<const v4u*>(xr + k0);
#pragma unroll
    for (int q = 0; q < NQ; ++q) st.w[q] = *reinterpret_cast<const v4u*>(wr[q] + k0);
    st.sc = *reinterpret_cast<const v4u*>(sr + k0);
}

// split 8 products s*w into bf16 hi (truncation) and lo (exact remainder)
__device__ __forceinline__ void split8(const v4u& w, const v4u& sc, v4u& hi, v4u& lo) {
    const uint32_t wa[4] = {w[0], w[1], w[2], w[3]}, sa[4] = {sc[0], sc[1], sc[2], sc[3]};
    uint32_t h[4], l[4];
    split_products8(wa, sa, h, l);
    hi = v4u{h[0], h[1], h[2], h[3]};
    lo = v4u{l[0], l[1], l[2], l[3]};
}

template <int NQ, int NS>
__global__ __launch_bounds__(kRThreads) void router_partial_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ scale,
    const uint16_t* __restrict__ w, int T, int H, int E, int slice_steps,
    float* __restrict__ partial, float* __restrict__ ss_partial) {
    constexpr int kMaxE = 32 * NQ, kMaxCT = kMaxE / 64;  // column tiles per wave
    // per stage: x tile [32][64], hi and lo tiles [32 NQ][64] (bf16)
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][kRT * kRK];
    __shared__ __attribute__((aligned(16))) uint16_t ws_hi[2][kMaxE * kRK];
    __shared__ __attribute__((aligned(16))) uint16_t ws_lo[2][kMaxE * kRK];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int t0 = blockIdx.x * kRT;
    const int nt = min(kRT, T - t0);
    const int n_ct = (E + 15) / 16;
    const int e_pad = n_ct * 16;
    const int nk = H / kRK, last = nk - 1;
    const int kb = blockIdx.y * slice_steps, ke = min(nk, kb + slice_steps);

    // staging sources: x chunk (row tid>>3, chunk tid&7); router rows tid>>3 + 32 q
    const int xr_row = tid >> 3, cc = tid & 7;
    const uint16_t* xr = x + (int64_t)(t0 + min(xr_row, nt - 1)) * H + cc * 8;
    const uint16_t* wr[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) wr[q] = w + (int64_t)min(xr_row + 32 * q, E - 1) * H + cc * 8;
    const uint16_t* sr = scale + cc * 8;

    f32x4_t acc[2][kMaxCT];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < kMaxCT; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    float ss = 0.f;  // this thread's share of the slice's sum of squares of its token row
    int step = 0;  // steps multiplied so far (selects the LDS buffer)
    for (int c0 = kb; c0 < ke; c0 += NS) {
        RStage<NQ> st[NS];
#pragma unroll
        for (int i = 0; i < NS; ++i) r_load(st[i], xr, wr, sr, min(c0 + i, last) * kRK);
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            if (c0 + i < ke) {  // uniform
                const int buf = (step + i) & 1;
                *reinterpret_cast<v4u*>(&xs[buf][rswz(xr_row, cc)]) = st[i].x;
                {
                    float f[8];
                    unpack8(make_uint4(st[i].x[0], st[i].x[1], st[i].x[2], st[i].x[3]), f);
#pragma unroll
                    for (int k = 0; k < 8; ++k) ss += f[k] * f[k];
                }
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    const int r = xr_row + 32 * q;
                    if (r < e_pad) {
                        v4u hi, lo;
                        split8(st[i].w[q], st[i].sc, hi, lo);
                        if (r >= E) hi = lo = v4u{0u, 0u, 0u, 0u};
                        *reinterpret_cast<v4u*>(&ws_hi[buf][rswz(r, cc)]) = hi;
                        *reinterpret_cast<v4u*>(&ws_lo[buf][rswz(r, cc)]) = lo;
                    }
                }
                __syncthreads();
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const int c = s * 4 + (lane >> 4);
                    bf16x8_t af[2];
#pragma unroll
                    for (int ii = 0; ii < 2; ++ii)
                        af[ii] = *reinterpret_cast<const bf16x8_t*>(&xs[buf][rswz(ii * 16 + (lane & 15), c)]);
#pragma unroll
                    for (int j = 0; j < kMaxCT; ++j) {
                        const int ct = wave + 4 * j;
                        if (ct < n_ct) {
                            const int r = ct * 16 + (lane & 15);
                            const bf16x8_t bh = *reinterpret_cast<const bf16x8_t*>(&ws_hi[buf][rswz(r, c)]);
                            const bf16x8_t bl = *reinterpret_cast<const bf16x8_t*>(&ws_lo[buf][rswz(r, c)]);
#pragma unroll
                            for (int ii = 0; ii < 2; ++ii) {
                                acc[ii][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ii], bh, acc[ii][j], 0, 0, 0);
                                acc[ii][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ii], bl, acc[ii][j], 0, 0, 0);
                            }
                        }
                    }
                }
            }
        }
        step += NS;
    }

    // the row's sum of squares over the slice: the 8 threads of a row are
    // consecutive lanes (tid & 7), added in a fixed order
    ss += __shfl_xor(ss, 1, kWave);
    ss += __shfl_xor(ss, 2, kWave);
    ss += __shfl_xor(ss, 4, kWave);
    if (cc == 0 && xr_row < nt) ss_partial[(int64_t)blockIdx.y * T + t0 + xr_row] = ss;

    float* out = partial + (int64_t)blockIdx.y * T * E;
#pragma unroll
    for (int j = 0; j < kMaxCT; ++j) {
        const int ct = wave + 4 * j;
        const int e = ct * 16 + (lane & 15);
        if (ct < n_ct && e < E) {
#pragma unroll
            for (int ii = 0; ii < 2; ++ii)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int r = ii * 16 + (lane >> 4) * 4 + v;
                    if (r < nt) out[(int64_t)(t0 + r) * E + e] = acc[ii][j][v];
                }
        }
    }
}

}  // namespace

__global__ __launch_bounds__(256) void router_finish_kernel(
    const float* __restrict__ partial, const float* __restrict__ ss_partial, int S,
    const float* __restrict__ bias, const float* __restrict__ pes, int T, int H, int E, int K,
    float eps, float inv_sqrt_h, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;  // uniform per wavefront
    float lv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = lane + kWave * j;
        float a = 0.f;
        if (e < E)
            for (int sl = 0; sl < S; ++sl) a += partial[((int64_t)sl * T + t) * E + e];
        lv[j] = a;
    }
    float q = 0.f;  // sum of squares of x_t: the slices' shares, in slice order
    for (int sl = 0; sl < S; ++sl) q += ss_partial[(int64_t)sl * T + t];
    const float f = (1.0f / sqrtf(q / (float)H + eps)) * inv_sqrt_h;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = lane + kWave * j;
        lv[j] = lv[j] * f + ((bias && e < E) ? bias[e] : 0.f);
    }
    int ik[kMaxTopK];
    float wk[kMaxTopK];
    wave_topk_vals(lv, pes, E, K, lane, ik, wk);
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k)
        if (k < K && lane == k) {
            topk_idx[(int64_t)t * K + k] = ik[k];
            topk_w[(int64_t)t * K + k] = wk[k];
        }
}

RouterSplit router_split(int T, int H, int E) {
    const int n_tiles = (T + kRT - 1) / kRT;
    const int nk = H / kRK;
    const int ns = E <= 128 ? 6 : 3;
    // about two workgroups per CU; slices of at least ns K-steps
    int S = (512 + n_tiles - 1) / n_tiles;
    S = S < 1 ? 1 : S;
    const int max_s = (nk + ns - 1) / ns;
    S = S > max_s ? max_s : S;
    const int steps = (nk + S - 1) / S;
    RouterSplit r;
    r.slice_steps = steps;
    r.slices = (nk + steps - 1) / steps;
    return r;
}

hipError_t launch_router_mfma(const uint16_t* x, const uint16_t* scale, const uint16_t* w,
                              const float* bias, const float* pes, int T, int H, int E, int K,
                              float eps, int32_t* topk_idx, float* topk_w, float* partial,
                              hipStream_t stream) {
    const float inv_sqrt_h = (float)(1.0 / __builtin_sqrt((double)H));
    const RouterSplit rs = router_split(T, H, E);
    const dim3 grid((T + kRT - 1) / kRT, rs.slices);
    // partial: the slices' logit sums [S][T][E], then their sums of squares [S][T]
    float* ss_partial = partial + (int64_t)rs.slices * T * E;
    if (E <= 128)
        hipLaunchKernelGGL((router_partial_kernel<4, 6>), grid, dim3(kRThreads), 0, stream, x, scale,
                           w, T, H, E, rs.slice_steps, partial, ss_partial);
    else
        hipLaunchKernelGGL((router_partial_kernel<8, 3>), grid, dim3(kRThreads), 0, stream, x, scale,
                           w, T, H, E, rs.slice_steps, partial, ss_partial);
    hipLaunchKernelGGL(router_finish_kernel, dim3((T + 3) / 4), dim3(256), 0, stream, partial, ss_partial,
                       rs.slices, bias, pes, T, H, E, K, eps, inv_sqrt_h, topk_idx, topk_w);
    return hipGetLastError();
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
