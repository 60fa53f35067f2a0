// Weight-streaming kernels for small batches (decode) on gfx950.
//
// With a handful of tokens per expert the block is bound by reading the
// weights of the touched experts from HBM once. These kernels stream each
// weight row exactly once with wide non-temporal loads and dot it with the
// (few) token vectors staged in LDS, accumulating in fp32.
//
//   stream_gateup: one work item = 16 gate rows (and the 16 matching up rows)
//     of one routed expert, or of the dense MLP; writes the bf16 intermediate
//     gelu_tanh(gate . x) * (up . x) for every token routed to it.
//   stream_down: output-stationary. One workgroup owns 8 output features of y
//     and reads those 8 rows of every routed expert's down matrix and of the
//     dense down matrix, so the weighted combine (dense + sum over k in k
//     order, ONNX export card "Truthful graph contracts", row "MoE topology")
//     happens in the same kernel without a rows buffer and without atomics.
// int8 experts (int8 experts card, "How it works") are read as int8 and
// widened in registers; the per-row scale multiplies the dot product.
#include "common.h"
#include "kernels.h"
#include "../../include/moe.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kRowsGU = 16;  // gate rows per gate/up work item (4 per wavefront)
constexpr int kPassTok = 8;  // tokens per pass over the weights
constexpr int kRowsDown = 8; // output features per down workgroup
constexpr int kMaxIC = 16;   // expert_inter <= 1024 on this path
constexpr int kMaxDC = 16;   // dense_inter chunks per lane: dense_inter <= 4096

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 ld_nt16(const void* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_nt8(const void* p) {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    return make_uint2(v.x, v.y);
}

// 8 weights of row `w` at element offset `col` -> floats
template <bool INT8>
__device__ __forceinline__ void load_w8(const void* w, int64_t col, float* f) {
    if (INT8) {
        unpack8_i8(ld_nt8(reinterpret_cast<const int8_t*>(w) + col), f);
    } else {
        unpack8(ld_nt16(reinterpret_cast<const uint16_t*>(w) + col), f);
    }
}

// raw 8-weight chunk (16 bytes of bf16, or 8 bytes of int8 in .x/.y)
template <bool INT8>
__device__ __forceinline__ uint4 load_raw(const void* w, int64_t col) {
    if (INT8) {
        const uint2 v = ld_nt8(reinterpret_cast<const int8_t*>(w) + col);
        return make_uint4(v.x, v.y, 0u, 0u);
    }
    return ld_nt16(reinterpret_cast<const uint16_t*>(w) + col);
}
template <bool INT8>
__device__ __forceinline__ void unpack_raw(const uint4& v, float* f) {
    if (INT8) unpack8_i8(make_uint2(v.x, v.y), f);
    else unpack8(v, f);
}

__device__ __forceinline__ float dot8(const float* a, const float* b) {
    float s = a[0] * b[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) s += a[i] * b[i];
    return s;
}

// gate/up rows [r0, r0 + kRowsGU) of one weight matrix (gate rows, then up rows
// at +inter) against the tokens tok(0..n_rows); writes out[row p][r].
template <bool INT8>
__device__ void gateup_item(const StreamArgs& a, uint4* xs, const void* W, const float* Ws,
                            int inter, int r0, const int32_t* toks, int n_rows, uint16_t* out) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int half = lane >> 5, hl = lane & 31;
    const int hc8 = a.H >> 3;        // 8-element chunks per row
    const int nj = a.H >> 8;         // chunks per lane (32 lanes per row)
    const int64_t H = a.H;
    for (int pass = 0; pass < n_rows; pass += kPassTok) {
        const int nt = min(kPassTok, n_rows - pass);
        __syncthreads();
        for (int i = tid; i < nt * hc8; i += kThreads) {
            const int n = i / hc8, c = i - n * hc8;
            const int64_t tok = toks ? toks[pass + n] : (int64_t)(pass + n);
            xs[i] = reinterpret_cast<const uint4*>(a.x + tok * H)[c];
        }
        __syncthreads();
#pragma unroll 1
        for (int q = 0; q < kRowsGU / 4; q += 2) {
            const int ra = r0 + wave * (kRowsGU / 4) + q, rb = ra + 1;
            // lanes 0..31: gate rows; lanes 32..63: the matching up rows
            const int64_t rowa = half ? (int64_t)inter + ra : ra;
            const int64_t rowb = half ? (int64_t)inter + rb : rb;
            float acc_a[kPassTok], acc_b[kPassTok];
#pragma unroll
            for (int n = 0; n < kPassTok; ++n) acc_a[n] = acc_b[n] = 0.f;
#pragma unroll 4
            for (int j = 0; j < nj; ++j) {
                const int c = hl + 32 * j;
                float wa[8], wb[8];
                load_w8<INT8>(W, rowa * H + c * 8, wa);
                load_w8<INT8>(W, rowb * H + c * 8, wb);
#pragma unroll
                for (int n = 0; n < kPassTok; ++n) {
                    if (n < nt) {
                        float xf[8];
                        unpack8(xs[n * hc8 + c], xf);
                        acc_a[n] += dot8(wa, xf);
                        acc_b[n] += dot8(wb, xf);
                    }
                }
            }
            float sga = 1.f, sua = 1.f, sgb = 1.f, sub = 1.f;
            if (INT8) {
                sga = Ws[ra]; sua = Ws[inter + ra];
                sgb = Ws[rb]; sub = Ws[inter + rb];
            }
            float ha = 0.f, hb = 0.f;
#pragma unroll
            for (int n = 0; n < kPassTok; ++n) {
                if (n < nt) {
                    const float va = wave_sum<32>(acc_a[n]);
                    const float vb = wave_sum<32>(acc_b[n]);
                    // every lane of a half now holds its row's dot; swap halves
                    const float oa = __shfl_xor(va, 32, kWave);
                    const float ob = __shfl_xor(vb, 32, kWave);
                    if (lane == n) ha = gelu_tanh(va * sga) * (oa * sua);
                    if (lane == 16 + n) hb = gelu_tanh(vb * sgb) * (ob * sub);
                }
            }
            if (lane < nt) out[(int64_t)(pass + lane) * inter + ra] = f32_to_bf16(ha);
            if (lane >= 16 && lane < 16 + nt) out[(int64_t)(pass + lane - 16) * inter + rb] = f32_to_bf16(hb);
        }
    }
}

template <bool INT8>
__global__ __launch_bounds__(kThreads) void stream_gateup_kernel(StreamArgs a) {
    extern __shared__ uint4 xs[];  // [kPassTok][H/8]
    const int gpe = a.I / kRowsGU;
    const int expert_items = a.max_active * gpe;
    const int b = blockIdx.x;
    if (b < expert_items) {
        const int slot = b / gpe, g = b - slot * gpe;
        if (slot >= *a.n_active) return;
        const int e = a.active[slot];
        const int p0 = a.offsets[e], n = a.offsets[e + 1] - p0;
        const int64_t wstride = (int64_t)2 * a.I * a.H;
        const void* W = INT8 ? (const void*)((const int8_t*)a.gu + e * wstride)
                             : (const void*)((const uint16_t*)a.gu + e * wstride);
        const float* Ws = INT8 ? a.gu_scale + (int64_t)e * 2 * a.I : nullptr;
        gateup_item<INT8>(a, xs, W, Ws, a.I, g * kRowsGU, a.perm_token + p0, n,
                          a.h + (int64_t)p0 * a.I);
    } else {
        const int g = b - expert_items;
        gateup_item<false>(a, xs, a.dgu, nullptr, a.Id, g * kRowsGU, nullptr, a.T, a.hd);
    }
}

template <bool INT8>
__global__ __launch_bounds__(kThreads) void stream_down_kernel(StreamArgs a) {
    __shared__ float part[MOE_STREAM_MAX_TOKENS * MOE_MAX_TOPK][kRowsDown];
    __shared__ float dpart[4][MOE_STREAM_MAX_TOKENS][kRowsDown];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int sub = lane & 7, rl = lane >> 3;
    const int h0 = blockIdx.x * kRowsDown;
    const int64_t row = h0 + rl;

    if (a.max_active > 0) {
        const int na = *a.n_active;
        const int ic = a.I >> 6;  // chunks per lane: I/8 chunks over 8 lanes
        for (int slot = wave; slot < na; slot += 4) {
            const int e = a.active[slot];
            const int64_t wbase = ((int64_t)e * a.H + row) * a.I;
            uint4 w[kMaxIC];  // raw weights: 8 bf16, or 8 int8 in .x/.y
#pragma unroll
            for (int j = 0; j < kMaxIC; ++j)
                if (j < ic) w[j] = load_raw<INT8>(a.dw, wbase + (int64_t)(sub + 8 * j) * 8);
            const float sc = INT8 ? a.dw_scale[(int64_t)e * a.H + row] : 1.f;
            const int p0 = a.offsets[e], p1 = a.offsets[e + 1];
            for (int p = p0; p < p1; ++p) {
                const uint4* hr = reinterpret_cast<const uint4*>(a.h + (int64_t)p * a.I);
                float acc = 0.f;
#pragma unroll
                for (int j = 0; j < kMaxIC; ++j)
                    if (j < ic) {
                        float hf[8], wf[8];
                        unpack8(hr[sub + 8 * j], hf);
                        unpack_raw<INT8>(w[j], wf);
                        acc += dot8(wf, hf);
                    }
                acc += __shfl_xor(acc, 1, kWave);
                acc += __shfl_xor(acc, 2, kWave);
                acc += __shfl_xor(acc, 4, kWave);
                if (sub == 0) part[p][rl] = acc * sc;
            }
        }
    }
    {
        // dense down: wavefront w reads chunks sub + 8*(w + 4*j) of the 8 rows
        const int dc = a.Id >> 3;
        const int64_t dbase = row * a.Id;
        uint4 w[kMaxDC];
#pragma unroll
        for (int j = 0; j < kMaxDC; ++j) {
            const int c = sub + 8 * (wave + 4 * j);
            if (c < dc) w[j] = load_raw<false>(a.ddw, dbase + (int64_t)c * 8);
        }
        for (int t = 0; t < a.T; ++t) {
            const uint4* hr = reinterpret_cast<const uint4*>(a.hd + (int64_t)t * a.Id);
            float acc = 0.f;
#pragma unroll
            for (int j = 0; j < kMaxDC; ++j) {
                const int c = sub + 8 * (wave + 4 * j);
                if (c < dc) {
                    float hf[8], wf[8];
                    unpack8(hr[c], hf);
                    unpack8(w[j], wf);
                    acc += dot8(wf, hf);
                }
            }
            acc += __shfl_xor(acc, 1, kWave);
            acc += __shfl_xor(acc, 2, kWave);
            acc += __shfl_xor(acc, 4, kWave);
            if (sub == 0) dpart[wave][t][rl] = acc;
        }
    }
    __syncthreads();
    for (int i = tid; i < a.T * kRowsDown; i += kThreads) {
        const int t = i / kRowsDown, r = i - t * kRowsDown;
        float v = dpart[0][t][r] + dpart[1][t][r] + dpart[2][t][r] + dpart[3][t][r];
        if (a.max_active > 0) {
            for (int k = 0; k < a.K; ++k) {
                const int q = a.inv_row[(int64_t)t * a.K + k];
                v += a.perm_w[q] * part[q][r];
            }
        }
        a.y[(int64_t)t * a.H + h0 + r] = f32_to_bf16(v);
    }
}

}  // namespace

hipError_t launch_stream_gateup(const StreamArgs& a, bool int8, hipStream_t stream) {
    const int blocks = a.max_active * (a.I / kRowsGU) + a.Id / kRowsGU;
    const size_t lds = (size_t)kPassTok * a.H * sizeof(uint16_t);
    if (int8)
        hipLaunchKernelGGL(stream_gateup_kernel<true>, dim3(blocks), dim3(kThreads), lds, stream, a);
    else
        hipLaunchKernelGGL(stream_gateup_kernel<false>, dim3(blocks), dim3(kThreads), lds, stream, a);
    return hipGetLastError();
}

hipError_t launch_stream_down(const StreamArgs& a, bool int8, hipStream_t stream) {
    const int blocks = a.H / kRowsDown;
    if (int8)
        hipLaunchKernelGGL(stream_down_kernel<true>, dim3(blocks), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(stream_down_kernel<false>, dim3(blocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace moe
