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

// ---- E4M3 (fp8 experts: the recipe page's fp8 variant) -------------------
// E4M3 in its OCP form without infinities: sign, 4 exponent bits (bias 7), 3
// mantissa bits; exponent field 0 holds the subnormals m 2^-9; the largest
// finite value is 448. The kernels carry E4M3 values as bf16 holding value *
// 2^-8 (half carriers) and fold 2^8 per operand into the scales.

// nearest E4M3 code of an fp32 value, ties to the even code, saturating at 448.
// Without branches: at or above 2^-6 the code is the float's exponent and top 3
// mantissa bits after a round-half-even add at bit 20 (a mantissa carry moves
// into the exponent field by itself), rebased from bias 127 to 7 and capped at
// code 0x7E (448); below 2^-6 it is the nearest multiple of 2^-9 (rint rounds
// half to even), code 8 being 2^-6 itself.
__device__ __forceinline__ uint32_t fp8_e4m3_code(float v) {
    const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
    const float a = fabsf(v);
    const uint32_t au = __float_as_uint(a);
    const uint32_t t = au + 0x7FFFFu + ((au >> 20) & 1u);
    const uint32_t cn = min((t >> 20) - (120u << 3), 0x7Eu);
    const uint32_t cs = (uint32_t)rintf(a * 512.f);
    return (a < 0.015625f ? cs : cn) | sign;
}

// the code of v / s (the division in fp32, as the quantisers define it), or 0
// when the row scale s is 0 (an all-zero row); without branches
__device__ __forceinline__ uint32_t fp8_e4m3_code_div(float v, float s) {
    const bool pos = s > 0.f;
    const uint32_t c = fp8_e4m3_code(v / (pos ? s : 1.f));
    return pos ? c : 0u;
}

// an E4M3 code's bits placed at the top of a half (sign to bit 15, exponent
// and mantissa to bits 7..13) are exactly its value * 2^-8, subnormals
// included (the exponent biases differ by 8): the half carrier of a code. (Code
// 0x7F, a NaN, never produced by the quantisers, would read as 480.)
__device__ __forceinline__ uint32_t fp8_as_f16_bits(uint32_t c) { return ((c & 0x80u) << 8) | ((c & 0x7Fu) << 7); }
// two E4M3 codes (bytes sh / 8 and sh / 8 + 1 of a word) -> a packed pair of half carriers
__device__ __forceinline__ uint32_t fp8pair_to_f16(uint32_t word, int sh) {
    const uint32_t p = ((word >> sh) & 0xFFu) | (((word >> sh) << 8) & 0xFF0000u);  // bytes to 0 and 2
    return ((p & 0x007F007Fu) << 7) | ((p & 0x00800080u) << 8);
}

// One wavefront quantises a bf16 row of nc 8-value chunks (nc <= 64 NC) to
// E4M3 per row: scale = max|x| / 448 (fp32, IEEE division), codes the nearest
// to x / scale, ties to even, written as half carriers to xq (xq == x allowed:
// the row is held in registers, all loads issued before any store). Returns
// the scale (0 for an all-zero row, whose codes are 0).
template <int NC>
__device__ __forceinline__ float fp8_quantize_row(const uint16_t* x, uint16_t* xq, int nc, int lane) {
    const uint4* src = reinterpret_cast<const uint4*>(x);
    uint4* dst = reinterpret_cast<uint4*>(xq);
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
        if (c < nc) {
            float f[8];
            unpack8(v[j], f);
            uint32_t o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t c0 = fp8_e4m3_code_div(f[2 * i], s);
                const uint32_t c1 = fp8_e4m3_code_div(f[2 * i + 1], s);
                o[i] = fp8_as_f16_bits(c0) | (fp8_as_f16_bits(c1) << 16);
            }
            dst[c] = make_uint4(o[0], o[1], o[2], o[3]);
        }
    }
    return s;
}

}  // namespace moe
