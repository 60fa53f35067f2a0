// Device helpers shared by the gfx950 kernels of the MoE FFN block.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

constexpr int kWave = 64;

// bfloat16 <-> fp32. Widening is exact; narrowing rounds to nearest even
// (finite inputs only: the block never produces inf/nan from finite weights).
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// 8 bf16 held in a uint4 -> 8 floats
__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
    f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
    f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}
// 8 int8 held in a uint2 -> 8 floats (exact)
__device__ __forceinline__ void unpack8_i8(const uint2& v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = (float)(int8_t)((v.x >> (8 * i)) & 0xFF);
#pragma unroll
    for (int i = 0; i < 4; ++i) f[4 + i] = (float)(int8_t)((v.y >> (8 * i)) & 0xFF);
}

// Products s*w of 8 bf16 pairs (packed two per word) are exact in fp32 (16
// significant bits); each is split into a bf16 hi (its truncation) and a bf16
// lo (the remainder, exactly representable), so hi + lo = s*w and two bf16 MFMAs
// against hi and lo accumulate the exact products in fp32.
__device__ __forceinline__ void split_products8(const uint32_t (&w)[4], const uint32_t (&s)[4],
                                                uint32_t (&hi)[4], uint32_t (&lo)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float p0 = bf16_lo(w[i]) * bf16_lo(s[i]);
        const float p1 = bf16_hi(w[i]) * bf16_hi(s[i]);
        const uint32_t h0 = __float_as_uint(p0) & 0xFFFF0000u, h1 = __float_as_uint(p1) & 0xFFFF0000u;
        const float r0 = p0 - __uint_as_float(h0), r1 = p1 - __uint_as_float(h1);
        hi[i] = (h0 >> 16) | h1;
        lo[i] = (__float_as_uint(r0) >> 16) | (__float_as_uint(r1) & 0xFFFF0000u);
    }
}

// GELU, tanh approximation ("gelu_pytorch_tanh"):
// 0.5 z (1 + tanh(u)), u = sqrt(2/pi) (z + 0.044715 z^3). Since
// 0.5 (1 + tanh(u)) = 1 / (1 + exp(-2u)), this is z / (1 + 2^(-2 u log2 e)),
// evaluated in fp32 with the hardware exp2 and reciprocal (a few ulp; the
// limits are exact: 2^t overflows to inf for very negative z, giving -0, and
// underflows to 0 for very positive z, giving z).
__device__ __forceinline__ float gelu_tanh(float z) {
    const float k = -2.0f * 0.7978845608028654f * 1.4426950408889634f;  // -2 sqrt(2/pi) log2(e)
    const float t = k * (z + 0.044715f * z * z * z);
    return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t));
}

// Butterfly reductions over the lanes [base, base + width) of a wavefront.
// The order of the additions is fixed, so results are bitwise reproducible.
template <int WIDTH>
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = WIDTH / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}
template <int WIDTH>
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = WIDTH / 2; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

// Workgroup barrier with no memory fence: the compiler moves no memory access
// across it, and the hardware waits for nothing (unlike __syncthreads, whose
// release waits for the wavefront's global loads and stores).
__device__ __forceinline__ void raw_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
// Barrier after this wavefront's LDS accesses have completed; its global
// loads and stores may still be in flight.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not waited on
    raw_barrier();
}

}  // namespace moe
