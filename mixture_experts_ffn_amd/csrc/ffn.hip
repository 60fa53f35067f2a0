// The layer's feed-forward norms around the MoE FFN block on gfx950.
//
// [INF2] "The architecture (a dual-path FFN)": the dense MLP and the MoE run in
// parallel and pass through four feed-forward layernorms; [ONNX] "Truthful
// graph contracts", row "MoE topology": post_ff_norm(dense + moe) + residual.
//   out = h + N_post(N_post_dense(dense) + N_post_moe(moe)),
// the branches run on x_d = bf16(N_pre_dense(h)) and x_m = bf16(N_pre_moe(h)),
// N_g(v) = v / sqrt(mean(v^2) + eps) * g per token (absent gain: no norm).
// Both kernels take one token row per workgroup: the row's sums of squares are
// workgroup reductions in a fixed order, and everything stays fp32 until the
// single rounding of each output.
#include "common.h"
#include "kernels.h"
#include "topk.h"

namespace moe {

namespace {

constexpr int kFT = 256;  // threads per token row
constexpr int kFWaves = kFT / kWave;

// the workgroup's sum of one value per thread (wavefront sums, then the
// wavefronts in order); every thread gets it
__device__ __forceinline__ float row_sum(float v, float* red) {
    v = wave_sum<kWave>(v);
    __syncthreads();  // red is free (a previous sum has been read)
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = v;
    __syncthreads();
    float s = red[0];
#pragma unroll
    for (int w = 1; w < kFWaves; ++w) s += red[w];
    return s;
}

__device__ __forceinline__ float inv_rms(float ss, int H, float eps) {
    return 1.0f / sqrtf(ss / (float)H + eps);
}

// x_d, x_m of token blockIdx.x (each only if its gain is given)
__global__ __launch_bounds__(kFT) void ffn_prenorm_kernel(const uint16_t* __restrict__ h, int H,
                                                          const uint16_t* __restrict__ gd,
                                                          const uint16_t* __restrict__ gm, float eps,
                                                          uint16_t* __restrict__ xd, uint16_t* __restrict__ xm) {
    __shared__ float red[kFWaves];
    const int64_t base = (int64_t)blockIdx.x * H;
    const uint4* row = reinterpret_cast<const uint4*>(h + base);
    const int n8 = H >> 3;
    float ss = 0.f;
    for (int c = threadIdx.x; c < n8; c += kFT) {
        float f[8];
        unpack8(row[c], f);
#pragma unroll
        for (int i = 0; i < 8; ++i) ss += f[i] * f[i];
    }
    const float rn = inv_rms(row_sum(ss, red), H, eps);
    for (int c = threadIdx.x; c < n8; c += kFT) {
        float f[8];
        unpack8(row[c], f);
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const uint16_t* g = b ? gm : gd;
            uint16_t* dst = b ? xm : xd;
            if (!g) continue;  // uniform
            float gv[8];
            unpack8(reinterpret_cast<const uint4*>(g)[c], gv);
            uint32_t o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                o[i] = pack_bf16x2(f[2 * i] * rn * gv[2 * i], f[2 * i + 1] * rn * gv[2 * i + 1]);
            reinterpret_cast<uint4*>(dst + base)[c] = make_uint4(o[0], o[1], o[2], o[3]);
        }
    }
}

// out for token t = blockIdx.x. The MoE branch of the token is the sum over
// k (in k order) of its rows rows[inv_row[t K + k]]: fp32 rows times topk_w
// (F32ROWS) or bf16 rows already weighted. LDS holds the fp32 dense and MoE
// rows, then their normed sum.
template <bool F32ROWS>
__global__ __launch_bounds__(kFT) void ffn_post_kernel(const uint16_t* __restrict__ h,
                                                       const float* __restrict__ dense,
                                                       const void* __restrict__ rows,
                                                       const int32_t* __restrict__ inv_row,
                                                       const float* __restrict__ topk_w, int H, int K,
                                                       const uint16_t* __restrict__ gpd,
                                                       const uint16_t* __restrict__ gpm,
                                                       const uint16_t* __restrict__ gp, float eps,
                                                       uint16_t* __restrict__ out) {
    extern __shared__ float buf[];  // [2][H]
    __shared__ float red[kFWaves];
    const int t = blockIdx.x;
    const int64_t base = (int64_t)t * H;
    int p[kMaxTopK];
    float wk[kMaxTopK];
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) {
        p[k] = inv_row[(int64_t)t * K + min(k, K - 1)];
        wk[k] = F32ROWS ? topk_w[(int64_t)t * K + min(k, K - 1)] : 1.f;
    }
    float ssd = 0.f, ssm = 0.f;
    for (int c = threadIdx.x * 4; c < H; c += kFT * 4) {
        const float4 d = *reinterpret_cast<const float4*>(dense + base + c);
        float m[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < kMaxTopK; ++k) {
            if (k < K) {
                float r[4];
                if (F32ROWS) {
                    const float4 v = *reinterpret_cast<const float4*>(
                        reinterpret_cast<const float*>(rows) + (int64_t)p[k] * H + c);
                    r[0] = v.x; r[1] = v.y; r[2] = v.z; r[3] = v.w;
                } else {
                    const uint2 v = *reinterpret_cast<const uint2*>(
                        reinterpret_cast<const uint16_t*>(rows) + (int64_t)p[k] * H + c);
                    r[0] = bf16_lo(v.x); r[1] = bf16_hi(v.x);
                    r[2] = bf16_lo(v.y); r[3] = bf16_hi(v.y);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) m[i] += F32ROWS ? wk[k] * r[i] : r[i];
            }
        }
        buf[c] = d.x; buf[c + 1] = d.y; buf[c + 2] = d.z; buf[c + 3] = d.w;
        ssd += d.x * d.x + d.y * d.y + d.z * d.z + d.w * d.w;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            buf[H + c + i] = m[i];
            ssm += m[i] * m[i];
        }
    }
    __syncthreads();  // the rows in LDS are read below by other threads than wrote them
    const float rnd = gpd ? inv_rms(row_sum(ssd, red), H, eps) : 1.f;
    const float rnm = gpm ? inv_rms(row_sum(ssm, red), H, eps) : 1.f;
    float sss = 0.f;
    for (int c = threadIdx.x; c < H; c += kFT) {
        const float gd = gpd ? bf16_to_f32(gpd[c]) : 1.f;
        const float gm = gpm ? bf16_to_f32(gpm[c]) : 1.f;
        const float s = buf[c] * rnd * gd + buf[H + c] * rnm * gm;
        buf[c] = s;
        sss += s * s;
    }
    const float rns = gp ? inv_rms(row_sum(sss, red), H, eps) : 1.f;
    for (int c = threadIdx.x; c < H; c += kFT) {
        const float g = gp ? bf16_to_f32(gp[c]) : 1.f;
        const float hv = bf16_to_f32(h[base + c]);
        out[base + c] = f32_to_bf16(hv + buf[c] * rns * g);
    }
}

}  // namespace

hipError_t launch_ffn_prenorm(const uint16_t* h, int T, int H, const uint16_t* gd, const uint16_t* gm, float eps,
                              uint16_t* xd, uint16_t* xm, hipStream_t stream) {
    if (T <= 0 || (!gd && !gm)) return hipSuccess;
    hipLaunchKernelGGL(ffn_prenorm_kernel, dim3(T), dim3(kFT), 0, stream, h, H, gd, gm, eps, xd, xm);
    return hipGetLastError();
}

hipError_t launch_ffn_post(const uint16_t* h, const float* dense, const void* rows, bool f32_rows,
                           const int32_t* inv_row, const float* topk_w, int T, int H, int K,
                           const uint16_t* gpd, const uint16_t* gpm, const uint16_t* gp, float eps, uint16_t* out,
                           hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    const size_t lds = (size_t)2 * H * sizeof(float);
    if (f32_rows)
        hipLaunchKernelGGL(ffn_post_kernel<true>, dim3(T), dim3(kFT), lds, stream, h, dense, rows, inv_row, topk_w,
                           H, K, gpd, gpm, gp, eps, out);
    else
        hipLaunchKernelGGL(ffn_post_kernel<false>, dim3(T), dim3(kFT), lds, stream, h, dense, rows, inv_row, topk_w,
                           H, K, gpd, gpm, gp, eps, out);
    return hipGetLastError();
}

}  // namespace moe
