// The layer's feed-forward norms around the MoE FFN block on gfx950.
//
// [INF2] "The architecture (a dual-path FFN)": the dense MLP and the MoE run in
// parallel and pass through four feed-forward layernorms; [ONNX] "Truthful
// graph contracts", row "MoE topology": post_ff_norm(dense + moe) + residual.
//   out = h + N_post(N_post_dense(dense) + N_post_moe(moe)),
// the branches run on x_d = bf16(N_pre_dense(h)) and x_m = bf16(N_pre_moe(h)),
// N_g(v) = v / sqrt(mean(v^2) + eps) * g per token (absent gain: no norm).
// Both kernels take one token row per workgroup (hidden sizes up to kFMaxH):
// the row's sums of squares are workgroup reductions in a fixed order, and
// everything stays fp32 until the single rounding of each output.
#include "common.h"
#include "kernels.h"
#include "topk.h"

namespace moe {

namespace {

typedef float f4v __attribute__((ext_vector_type(4)));
typedef unsigned int u2v __attribute__((ext_vector_type(2)));

// A workgroup of NT threads per token row holds the row in registers, up to
// kFR four-value pieces a thread: hidden sizes up to 4 kFR NT. Small batches take
// 1024 threads a row (more loads in flight for few rows), larger ones 256 (more
// rows resident per CU).
constexpr int kFR = 4;
constexpr int kFMaxH = 4 * kFR * 1024;

// the workgroup's sums of two values per thread (wavefront sums, then the
// wavefronts in order); every thread gets them
template <int NT>
__device__ __forceinline__ float2 row_sum2(float a, float b, float2* red) {
    a = wave_sum<kWave>(a);
    b = wave_sum<kWave>(b);
    __syncthreads();  // red is free (a previous sum has been read)
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = make_float2(a, b);
    __syncthreads();
    float2 s = red[0];
#pragma unroll
    for (int w = 1; w < NT / kWave; ++w) {
        s.x += red[w].x;
        s.y += red[w].y;
    }
    return s;
}

__device__ __forceinline__ float inv_rms(float ss, int H, float eps) {
    return 1.0f / sqrtf(ss / (float)H + eps);
}

// x_d, x_m of token blockIdx.x (each only if its gain is given). Each thread
// holds its (at most kFR) four-value pieces of the row in registers: the row
// is read once.
template <int NT>
__global__ __launch_bounds__(NT) void ffn_prenorm_kernel(const uint16_t* __restrict__ h, int H,
                                                          const uint16_t* __restrict__ gd,
                                                          const uint16_t* __restrict__ gm, float eps,
                                                          uint16_t* __restrict__ xd, uint16_t* __restrict__ xm) {
    __shared__ float2 red[NT / kWave];
    const int64_t base = (int64_t)blockIdx.x * H;
    const uint2* row = reinterpret_cast<const uint2*>(h + base);
    const int n4 = H >> 2;
    // the row's pieces, and both gains' (with few rows, 1024 threads a row,
    // loaded before the reduction; with many where they are used)
    constexpr bool kEarly = NT >= 1024;
    uint2 v[kFR], gv[kFR][2];
    auto load_gains = [&](int q) {
        const int c = threadIdx.x + q * NT;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const uint16_t* g = b ? gm : gd;
            gv[q][b] = (g && c < n4) ? reinterpret_cast<const uint2*>(g)[c] : make_uint2(0u, 0u);
        }
    };
    float ss = 0.f;
#pragma unroll
    for (int q = 0; q < kFR; ++q) {
        const int c = threadIdx.x + q * NT;
        v[q] = c < n4 ? row[c] : make_uint2(0u, 0u);
        if (kEarly) load_gains(q);
        const float f0 = bf16_lo(v[q].x), f1 = bf16_hi(v[q].x), f2 = bf16_lo(v[q].y), f3 = bf16_hi(v[q].y);
        ss += f0 * f0 + f1 * f1 + f2 * f2 + f3 * f3;
    }
    const float rn = inv_rms(row_sum2<NT>(ss, 0.f, red).x, H, eps);
#pragma unroll
    for (int q = 0; q < kFR; ++q) {
        const int c = threadIdx.x + q * NT;
        if (c >= n4) continue;
        if (!kEarly) load_gains(q);
        const float f0 = bf16_lo(v[q].x), f1 = bf16_hi(v[q].x), f2 = bf16_lo(v[q].y), f3 = bf16_hi(v[q].y);
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const uint16_t* g = b ? gm : gd;
            uint16_t* dst = b ? xm : xd;
            if (!g) continue;  // uniform
            const uint2 gq = gv[q][b];
            reinterpret_cast<uint2*>(dst + base)[c] =
                make_uint2(pack_bf16x2(f0 * rn * bf16_lo(gq.x), f1 * rn * bf16_hi(gq.x)),
                           pack_bf16x2(f2 * rn * bf16_lo(gq.y), f3 * rn * bf16_hi(gq.y)));
        }
    }
}

// out for token t = blockIdx.x. The MoE branch of the token is the sum over
// k (in k order) of its rows rows[inv_row[t K + k]]: fp32 rows times topk_w
// (F32ROWS) or bf16 rows already weighted. Each thread keeps its (at most
// FR) four-value pieces of the dense and MoE rows in registers; the two
// branches' sums of squares are one reduction, their normed sum's another.
template <int NT, int FR, bool F32ROWS>
__global__ __launch_bounds__(NT) void ffn_post_kernel(const uint16_t* __restrict__ h,
                                                       const float* __restrict__ dense,
                                                       const void* __restrict__ rows,
                                                       const int32_t* __restrict__ inv_row,
                                                       const float* __restrict__ topk_w, int H, int K,
                                                       const uint16_t* __restrict__ gpd,
                                                       const uint16_t* __restrict__ gpm,
                                                       const uint16_t* __restrict__ gp, float eps,
                                                       uint16_t* __restrict__ out) {
    __shared__ float2 red[NT / kWave];
    const int t = blockIdx.x;
    const int64_t base = (int64_t)t * H;
    const int n4 = H >> 2;
    int p[kMaxTopK];
    float wk[kMaxTopK];
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) {
        p[k] = inv_row[(int64_t)t * K + min(k, K - 1)];
        wk[k] = F32ROWS ? topk_w[(int64_t)t * K + min(k, K - 1)] : 1.f;
    }
    // the gains and the residual row: with few rows (1024 threads a row) loaded
    // here, beside the branch rows, so that nothing after the reductions waits
    // on memory; with many rows where they are used (fewer registers, more
    // rows resident)
    constexpr bool kEarly = NT >= 1024;
    constexpr uint32_t kOne = 0x3F803F80u;  // two bf16 ones
    uint2 gdv[FR], gmv[FR], gv[FR], hv[FR];
    auto load_norm_gains = [&](int q) {
        const int c = min((int)threadIdx.x + q * NT, n4 - 1) * 4;
        gdv[q] = gpd ? *reinterpret_cast<const uint2*>(gpd + c) : make_uint2(kOne, kOne);
        gmv[q] = gpm ? *reinterpret_cast<const uint2*>(gpm + c) : make_uint2(kOne, kOne);
    };
    auto load_out_operands = [&](int q) {
        const int c = min((int)threadIdx.x + q * NT, n4 - 1) * 4;
        gv[q] = gp ? *reinterpret_cast<const uint2*>(gp + c) : make_uint2(kOne, kOne);
        hv[q] = *reinterpret_cast<const uint2*>(h + base + c);
    };
    if (kEarly) {
#pragma unroll
        for (int q = 0; q < FR; ++q) {
            load_norm_gains(q);
            load_out_operands(q);
        }
    }
    float d[FR][4], m[FR][4];
    float ssd = 0.f, ssm = 0.f;
#pragma unroll
    for (int q = 0; q < FR; ++q) {
        const int c4 = threadIdx.x + q * NT;
        const int c = min(c4, n4 - 1) * 4;  // past the row: a repeat of its last piece, never stored
        // the dense output and the expert rows are read once: non-temporal loads
        const f4v dv = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(dense + base + c));
        d[q][0] = dv.x; d[q][1] = dv.y; d[q][2] = dv.z; d[q][3] = dv.w;
#pragma unroll
        for (int i = 0; i < 4; ++i) m[q][i] = 0.f;
#pragma unroll
        for (int k = 0; k < kMaxTopK; ++k) {
            if (k < K) {
                float r[4];
                if (F32ROWS) {
                    const f4v v = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(
                        reinterpret_cast<const float*>(rows) + (int64_t)p[k] * H + c));
                    r[0] = v.x; r[1] = v.y; r[2] = v.z; r[3] = v.w;
                } else {
                    const u2v v = __builtin_nontemporal_load(reinterpret_cast<const u2v*>(
                        reinterpret_cast<const uint16_t*>(rows) + (int64_t)p[k] * H + c));
                    r[0] = bf16_lo(v.x); r[1] = bf16_hi(v.x);
                    r[2] = bf16_lo(v.y); r[3] = bf16_hi(v.y);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) m[q][i] += F32ROWS ? wk[k] * r[i] : r[i];
            }
        }
        if (c4 < n4) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ssd += d[q][i] * d[q][i];
                ssm += m[q][i] * m[q][i];
            }
        }
    }
    float rnd = 1.f, rnm = 1.f;
    if (gpd || gpm) {  // uniform
        const float2 ss = row_sum2<NT>(ssd, ssm, red);
        if (gpd) rnd = inv_rms(ss.x, H, eps);
        if (gpm) rnm = inv_rms(ss.y, H, eps);
    }
    float sss = 0.f;
#pragma unroll
    for (int q = 0; q < FR; ++q) {
        const int c4 = threadIdx.x + q * NT;
        if (!kEarly) load_norm_gains(q);
        const float gdf[4] = {bf16_lo(gdv[q].x), bf16_hi(gdv[q].x), bf16_lo(gdv[q].y), bf16_hi(gdv[q].y)};
        const float gmf[4] = {bf16_lo(gmv[q].x), bf16_hi(gmv[q].x), bf16_lo(gmv[q].y), bf16_hi(gmv[q].y)};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            d[q][i] = d[q][i] * rnd * gdf[i] + m[q][i] * rnm * gmf[i];  // the branches' sum
            if (c4 < n4) sss += d[q][i] * d[q][i];
        }
    }
    const float rns = gp ? inv_rms(row_sum2<NT>(sss, 0.f, red).x, H, eps) : 1.f;
#pragma unroll
    for (int q = 0; q < FR; ++q) {
        const int c4 = threadIdx.x + q * NT;
        if (c4 >= n4) continue;
        const int c = c4 * 4;
        if (!kEarly) load_out_operands(q);
        const float g[4] = {bf16_lo(gv[q].x), bf16_hi(gv[q].x), bf16_lo(gv[q].y), bf16_hi(gv[q].y)};
        const float hf[4] = {bf16_lo(hv[q].x), bf16_hi(hv[q].x), bf16_lo(hv[q].y), bf16_hi(hv[q].y)};
        *reinterpret_cast<uint2*>(out + base + c) =
            make_uint2(pack_bf16x2(hf[0] + d[q][0] * rns * g[0], hf[1] + d[q][1] * rns * g[1]),
                       pack_bf16x2(hf[2] + d[q][2] * rns * g[2], hf[3] + d[q][3] * rns * g[3]));
    }
}

}  // namespace

namespace {
// threads per token row for a launch of T rows of H values
int ffn_threads(int T, int H) { return (T >= 512 && H <= 4 * kFR * 256) ? 256 : 1024; }
}  // namespace

hipError_t launch_ffn_prenorm(const uint16_t* h, int T, int H, const uint16_t* gd, const uint16_t* gm, float eps,
                              uint16_t* xd, uint16_t* xm, hipStream_t stream) {
    if (T <= 0 || (!gd && !gm)) return hipSuccess;
    if (H > kFMaxH) return hipErrorInvalidValue;
    if (ffn_threads(T, H) == 256)
        hipLaunchKernelGGL(ffn_prenorm_kernel<256>, dim3(T), dim3(256), 0, stream, h, H, gd, gm, eps, xd, xm);
    else
        hipLaunchKernelGGL(ffn_prenorm_kernel<1024>, dim3(T), dim3(1024), 0, stream, h, H, gd, gm, eps, xd, xm);
    return hipGetLastError();
}

hipError_t launch_ffn_post(const uint16_t* h, const float* dense, const void* rows, bool f32_rows,
                           const int32_t* inv_row, const float* topk_w, int T, int H, int K,
                           const uint16_t* gpd, const uint16_t* gpm, const uint16_t* gp, float eps, uint16_t* out,
                           hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    if (H > kFMaxH) return hipErrorInvalidValue;
    // pieces a thread: the fewest that cover the row
#define MOE_FFN_POST(NT, FR, F32)                                                                              \
    hipLaunchKernelGGL((ffn_post_kernel<NT, FR, F32>), dim3(T), dim3(NT), 0, stream, h, dense, rows, inv_row, \
                       topk_w, H, K, gpd, gpm, gp, eps, out)
#define MOE_FFN_POST_FR(NT, F32)                            \
    do {                                                    \
        const int fr = (H + 4 * NT - 1) / (4 * NT);         \
        if (fr <= 1) MOE_FFN_POST(NT, 1, F32);              \
        else if (fr <= 2) MOE_FFN_POST(NT, 2, F32);         \
        else if (fr <= 3) MOE_FFN_POST(NT, 3, F32);         \
        else MOE_FFN_POST(NT, 4, F32);                      \
    } while (0)
    const bool small = ffn_threads(T, H) == 256;
    if (f32_rows) {
        if (small) MOE_FFN_POST_FR(256, true);
        else MOE_FFN_POST_FR(1024, true);
    } else {
        if (small) MOE_FFN_POST_FR(256, false);
        else MOE_FFN_POST_FR(1024, false);
    }
#undef MOE_FFN_POST_FR
#undef MOE_FFN_POST
    return hipGetLastError();
}

}  // namespace moe
