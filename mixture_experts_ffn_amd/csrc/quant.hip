// Per-row symmetric int8 quantisation of bf16 weights (int8 experts card,
// intro: "per-channel symmetric int8"; "How it works": the fused expert
// weights are quantised when the checkpoint is loaded).
// scale = max|w| / 127 in fp32 (IEEE division); q = round-half-even(w / scale)
// clamped to [-127, 127]; an all-zero row gets scale 0 and q 0.
#include "common.h"
#include "kernels.h"

namespace moe {

__global__ __launch_bounds__(256) void quantize_int8_kernel(const uint16_t* __restrict__ w,
                                                            int64_t rows, int cols,
                                                            int8_t* __restrict__ q,
                                                            float* __restrict__ scale) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + wave;
    if (r >= rows) return;
    const uint4* src = reinterpret_cast<const uint4*>(w + r * cols);
    const int nc = cols >> 3;
    float amax = 0.f;
    for (int c = lane; c < nc; c += kWave) {
        float f[8];
        unpack8(src[c], f);
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
    }
    amax = wave_max<kWave>(amax);
    const float s = amax / 127.0f;
    if (lane == 0) scale[r] = s;
    uint2* dst = reinterpret_cast<uint2*>(q + r * cols);
    for (int c = lane; c < nc; c += kWave) {
        float f[8];
        unpack8(src[c], f);
        uint32_t b[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float v = 0.f;
            if (s > 0.f) v = fminf(fmaxf(rintf(f[i] / s), -127.f), 127.f);
            b[i] = (uint32_t)(int32_t)v & 0xFFu;
        }
        dst[c] = make_uint2(b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24),
                            b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24));
    }
}

hipError_t launch_quantize_int8(const uint16_t* w, int64_t rows, int cols, int8_t* q, float* scale,
                                hipStream_t stream) {
    const int64_t blocks = (rows + 3) / 4;
    hipLaunchKernelGGL(quantize_int8_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, w, rows,
                       cols, q, scale);
    return hipGetLastError();
}

// ---- E4M3 (the recipe page's fp8 variant: E4M3 weights, activations
// quantised per token at run time). scale = max|v| / 448 in fp32 (IEEE
// division); code = nearest E4M3 of v / scale, ties to the even code; an
// all-zero row gets scale 0 and codes 0.

// weights: one wavefront a row of a bf16 [rows, cols] matrix -> codes + scale
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const uint16_t* __restrict__ w, int64_t rows,
                                                           int cols, uint8_t* __restrict__ q,
                                                           float* __restrict__ scale) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + wave;
    if (r >= rows) return;
    const uint4* src = reinterpret_cast<const uint4*>(w + r * cols);
    const int nc = cols >> 3;
    float amax = 0.f;
    for (int c = lane; c < nc; c += kWave) {
        float f[8];
        unpack8(src[c], f);
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
    }
    amax = wave_max<kWave>(amax);
    const float s = amax / 448.0f;
    if (lane == 0) scale[r] = s;
    uint2* dst = reinterpret_cast<uint2*>(q + r * cols);
    for (int c = lane; c < nc; c += kWave) {
        float f[8];
        unpack8(src[c], f);
        uint32_t b[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) b[i] = fp8_e4m3_code_div(f[i], s);
        dst[c] = make_uint2(b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24),
                            b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24));
    }
}

// activations for the E4M3 MFMAs: one wavefront a row of a bf16 [rows, cols]
// matrix, the row held in registers -> the row's E4M3 codes, one byte each, in
// a row of ldq >= cols bytes whose tail past cols is zero (so that a K-step of
// 128 codes may run past cols and add nothing), its scale, and (mul_out)
// mul_in[r] * scale[r], the factor the down projection's rows take
template <int NC>
__global__ __launch_bounds__(256) void act_quant_fp8_bytes_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                                  int cols, uint8_t* __restrict__ q, int ldq,
                                                                  float* __restrict__ scale,
                                                                  const float* __restrict__ mul_in,
                                                                  float* __restrict__ mul_out) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + wave;
    if (r >= rows) return;
    const int nc = cols >> 3, ncq = ldq >> 3;
    const uint4* src = reinterpret_cast<const uint4*>(x + r * cols);
    uint2* dst = reinterpret_cast<uint2*>(q + r * ldq);
    uint4 v[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j) v[j] = src[min(lane + j * kWave, nc - 1)];  // clamped: same max
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        float f[8];
        unpack8(v[j], f);
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
    }
    amax = wave_max<kWave>(amax);
    const float s = amax / 448.0f;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        const int c = lane + j * kWave;
        if (c < ncq) {
            uint32_t o[2] = {0u, 0u};
            if (c < nc) {
                float f[8];
                unpack8(v[j], f);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    o[i >> 2] |= fp8_e4m3_code_div(f[i], s) << (8 * (i & 3));
            }
            dst[c] = make_uint2(o[0], o[1]);
        }
    }
    if (lane == 0) {
        scale[r] = s;
        if (mul_out) mul_out[r] = mul_in[r] * s;
    }
}

hipError_t launch_quantize_fp8(const uint16_t* w, int64_t rows, int cols, uint8_t* q, float* scale,
                               hipStream_t stream) {
    const int64_t blocks = (rows + 3) / 4;
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(quantize_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, w, rows, cols, q,
                       scale);
    return hipGetLastError();
}

hipError_t launch_act_quant_fp8_bytes(const uint16_t* x, int64_t rows, int cols, uint8_t* q, int ldq, float* scale,
                                      const float* mul_in, float* mul_out, hipStream_t stream) {
    const int64_t blocks = (rows + 3) / 4;
    if (blocks <= 0) return hipSuccess;
    const int nc = (ldq / 8 + kWave - 1) / kWave;  // 8-value chunks a lane, the zero tail included
#define LAUNCH(N)                                                                                              \
    do {                                                                                                       \
        hipLaunchKernelGGL(act_quant_fp8_bytes_kernel<N>, dim3((unsigned)blocks), dim3(256), 0, stream, x, rows, \
                           cols, q, ldq, scale, mul_in, mul_out);                                              \
        return hipGetLastError();                                                                              \
    } while (0)
    if (nc <= 2) LAUNCH(2);
    if (nc <= 4) LAUNCH(4);
    if (nc <= 6) LAUNCH(6);
    if (nc <= 8) LAUNCH(8);
    if (nc <= 16) LAUNCH(16);
    if (nc <= 33) LAUNCH(33);
#undef LAUNCH
    return hipErrorInvalidValue;  // ldq <= 16896
}

}  // namespace moe
