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

}  // namespace moe
