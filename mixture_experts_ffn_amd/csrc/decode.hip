// Small-batch (decode) path of the MoE FFN block on gfx950.
//
// With a handful of tokens per expert the block is bound by reading the
// touched experts' weights from HBM once. The weights are in the tiled layout
// (16 rows x 64 k per tile, lane l of a wavefront owning row l % 16, k
// 16 (l / 16) .. + 16 of each tile), so a wavefront streams a 16-row block of
// a matrix as contiguous 1 KB loads; each lane dots its 16-value pieces with
// the matching x values (from LDS) and four lanes' partial sums make a row.
// Five launches, each filling the chip (the dense MLP's items ride along in
// K1, K2 and K4 when with_dense is set):
//
//   K1 decode_front: router logits (two experts per wavefront) side by side
//      with the dense MLP's gate/up tiles, whose K range is split over
//      kDenseSplit workgroups (fp32 partial sums); both only need x.
//   K2 decode_route: one workgroup: softmax/top-k of every token (ONNX export
//      card, "Truthful graph contracts", row "Router") and the grouping of the
//      routed pairs by expert (counts, offsets, grouped rows, inverse rows,
//      list of touched experts); the other workgroups add the dense partial
//      sums and form the dense intermediate gelu_tanh(gate) * up.
//   K3 decode_experts_gateup: 16 gate columns (+ the 16 matching up columns)
//      of one touched expert per workgroup, K split over its 4 wavefronts;
//      every weight byte is read exactly once with wide non-temporal loads
//      issued before anything waits, then dotted with the expert's tokens
//      staged in LDS.
//   K4 decode_down: one 16-row tile of a touched expert's down matrix per
//      wavefront (fp32 partial rows per routed pair), and the dense down
//      matrix with K split over a workgroup's wavefronts.
//   K5 decode_combine: y = dense + sum_k w_k * expert_k in k order (row "MoE
//      topology"), without atomics.
// int8 experts (int8 experts card, "How it works") are read as int8, widened
// exactly in registers, and their per-row scale multiplies the dot product.
#include "common.h"
#include "kernels.h"
#include "topk.h"
#include "../../include/moe.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kPass = 4;           // tokens staged per pass
constexpr int kDensePass = 8;      // tokens per pass of the dense gate/up partial sums
constexpr int kRouterExperts = 8;  // experts per router work item: 2 per wavefront
constexpr int kRouteThreads = 1024;
constexpr int kMaxPairs = MOE_STREAM_MAX_TOKENS * MOE_MAX_TOPK;

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
// 8 weights at element offset `col` of a weight matrix: 16 bytes of bf16, or
// 8 bytes of int8 kept in .x/.y
template <bool INT8>
__device__ __forceinline__ uint4 load_w8(const void* w, int64_t col) {
    if (INT8) {
        const uint2 v = ld_nt8(reinterpret_cast<const int8_t*>(w) + col);
        return make_uint4(v.x, v.y, 0u, 0u);
    }
    return ld_nt16(reinterpret_cast<const uint16_t*>(w) + col);
}
template <bool INT8>
__device__ __forceinline__ void unpack_w8(const uint4& v, float* f) {
    if (INT8) unpack8_i8(make_uint2(v.x, v.y), f);
    else unpack8(v, f);
}
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

// acc + a.lo*b.lo + a.hi*b.hi on packed bf16 pairs (v_dot2c_f32_bf16, fp32
// accumulation; no unpacking of either operand)
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), acc, false);
}
__device__ __forceinline__ float dot8_bf16(const uint4& a, const uint4& b, float acc) {
    acc = dot2(a.x, b.x, acc);
    acc = dot2(a.y, b.y, acc);
    acc = dot2(a.z, b.z, acc);
    return dot2(a.w, b.w, acc);
}
// 8 int8 (in .x/.y) -> 8 bf16 (exact: |q| <= 127 fits the bf16 significand)
__device__ __forceinline__ uint4 i8x8_to_bf16(const uint4& v) {
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t word = q < 2 ? v.x : v.y;
        const int sh = (q & 1) * 16;
        const float lo = (float)(int8_t)((word >> sh) & 0xFF);
        const float hi = (float)(int8_t)((word >> (sh + 8)) & 0xFF);
        o[q] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}
// weights as packed bf16, whatever their storage
template <bool INT8>
__device__ __forceinline__ uint4 as_bf16(const uint4& v) {
    if (INT8) return i8x8_to_bf16(v);
    return v;
}

__device__ __forceinline__ float dot8(const float* a, const float* b) {
    float s = a[0] * b[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) s += a[i] * b[i];
    return s;
}

// Stage x rows tok(pass .. pass+nt) into LDS as [kPass][H/8] 16-byte chunks.
// Every load is unconditional (indices clamped into range) so that all of them
// are in flight together; only the LDS stores are predicated.
template <int NJ>
__device__ __forceinline__ void stage_x(const uint16_t* __restrict__ x, int H, const int32_t* toks,
                                        int pass, int nt, uint4* xs) {
    const int hc8 = H >> 3;
    const int n = nt * hc8;
    constexpr int kPer = (kPass * 32 * NJ + kThreads - 1) / kThreads;  // chunks per thread
    int64_t tok[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int i = min((int)threadIdx.x + q * kThreads, n - 1);
        const int r = i / hc8;
        tok[q] = toks ? (int64_t)toks[pass + r] : (int64_t)(pass + r);
    }
    uint4 v[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int i = min((int)threadIdx.x + q * kThreads, n - 1);
        const int c = i - (i / hc8) * hc8;
        v[q] = reinterpret_cast<const uint4*>(x + tok[q] * H)[c];
    }
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int i = threadIdx.x + q * kThreads;
        if (i < n) xs[i] = v[q];
    }
}

// Copy n (1 <= n <= KPER * 256) contiguous 16-byte chunks into LDS; loads are
// unconditional (indices clamped into range) so that all are in flight.
template <int KPER>
__device__ __forceinline__ void stage_rows(const uint4* __restrict__ src, int n, uint4* dst) {
    uint4 v[KPER];
#pragma unroll
    for (int q = 0; q < KPER; ++q) v[q] = src[min((int)threadIdx.x + q * kThreads, n - 1)];
#pragma unroll
    for (int q = 0; q < KPER; ++q) {
        const int i = (int)threadIdx.x + q * kThreads;
        if (i < n) dst[i] = v[q];
    }
}

// Rows of a pass staged through LDS in two halves, so that other loads can be
// issued between them. rows_load: chunk i = tid + 256 q (i < n = nt * len8,
// n >= 1) is 16-byte piece i % len8, from element k0, of row r = i / len8 of
// the pass, which is src row toks[pass + r] (or pass + r without toks);
// indices are clamped into range, so every load is unconditional and all are
// in flight together. rows_store writes them to LDS as [nt][len8] chunks.
template <int KPER>
__device__ __forceinline__ void rows_load(const uint16_t* __restrict__ src, int64_t stride, int k0, int len8,
                                          const int32_t* toks, int pass, int n, uint4 (&v)[KPER]) {
#pragma unroll
    for (int q = 0; q < KPER; ++q) {
        const int i = min((int)threadIdx.x + q * kThreads, n - 1);
        const int r = i / len8;
        const int64_t row = toks ? (int64_t)toks[pass + r] : (int64_t)(pass + r);
        v[q] = reinterpret_cast<const uint4*>(src + row * stride + k0)[i - r * len8];
    }
}
template <int KPER>
__device__ __forceinline__ void rows_store(const uint4 (&v)[KPER], int n, uint4* xs) {
#pragma unroll
    for (int q = 0; q < KPER; ++q) {
        const int i = (int)threadIdx.x + q * kThreads;
        if (i < n) xs[i] = v[q];
    }
}

// 16 int8 (one tiled-layout piece) -> two groups of 8 bf16 (exact)
__device__ __forceinline__ void i8x16_to_bf16(const uint4& v, uint4& lo, uint4& hi) {
    lo = i8x8_to_bf16(make_uint4(v.x, v.y, 0u, 0u));
    hi = i8x8_to_bf16(make_uint4(v.z, v.w, 0u, 0u));
}

// One K-step of a lane's piece of a tile (bf16: two 16-byte halves, 8 k each;
// int8: one 16-byte piece, 16 k) dotted with the 16 matching x values.
template <bool INT8>
__device__ __forceinline__ float piece_dot(const uint4 (&w)[INT8 ? 1 : 2], const uint16_t* xp,
                                           float acc) {
    const uint4 x0 = *reinterpret_cast<const uint4*>(xp);
    const uint4 x1 = *reinterpret_cast<const uint4*>(xp + 8);
    if (INT8) {
        uint4 lo, hi;
        i8x16_to_bf16(w[0], lo, hi);
        acc = dot8_bf16(lo, x0, acc);
        return dot8_bf16(hi, x1, acc);
    }
    acc = dot8_bf16(w[0], x0, acc);
    return dot8_bf16(w[INT8 ? 0 : 1], x1, acc);
}

// sum of the four lanes holding one row of a tile (lanes r, r+16, r+32, r+48)
__device__ __forceinline__ float tile_row_sum(float v) {
    v += __shfl_xor(v, 16, kWave);
    return v + __shfl_xor(v, 32, kWave);
}

template <bool INT8>
constexpr int kTileBytes = INT8 ? 1024 : 2048;

// Load steps kt0 .. kt0 + NS - 1 (clamped to the last step nk - 1) of this
// lane's pieces of a tile whose step 0 starts at `tile`; all loads issued at once.
template <int NS, bool INT8>
__device__ __forceinline__ void tile_load(const char* tile, int kt0, int nk, int lane,
                                          uint4 (&w)[NS][INT8 ? 1 : 2]) {
    const char* p = tile + lane * 16;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int64_t off = (int64_t)min(kt0 + s, nk - 1) * kTileBytes<INT8>;
        w[s][0] = ld_nt16(p + off);
        if (!INT8) w[s][INT8 ? 0 : 1] = ld_nt16(p + off + 1024);
    }
}

// tile_load of two tiles at once, their loads interleaved step by step (so
// that step s of both has landed once 2 (s + 1) of them have).
template <int NS, bool INT8>
__device__ __forceinline__ void tile_load2(const char* ta, const char* tb, int kt0, int nk, int lane,
                                           uint4 (&wa)[NS][INT8 ? 1 : 2], uint4 (&wb)[NS][INT8 ? 1 : 2]) {
    const char* pa = ta + lane * 16;
    const char* pb = tb + lane * 16;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int64_t off = (int64_t)min(kt0 + s, nk - 1) * kTileBytes<INT8>;
        wa[s][0] = ld_nt16(pa + off);
        if (!INT8) wa[s][INT8 ? 0 : 1] = ld_nt16(pa + off + 1024);
        wb[s][0] = ld_nt16(pb + off);
        if (!INT8) wb[s][INT8 ? 0 : 1] = ld_nt16(pb + off + 1024);
    }
}

// Gate/up of 16 h columns (gate tile hc of a tiled [2*inter, H] matrix and the
// matching up tile inter/16 + hc) against tokens tok(0 .. n_rows):
// out[p][16 hc + r] = gelu_tanh(gate_r . x_p) * (up_r . x_p). Wavefront w takes
// K-steps [w NS, (w + 1) NS) of both tiles (NS = H / 256); the four partial
// sums of a column are added in wavefront order through LDS.
template <int NS, bool INT8>
__device__ __forceinline__ void gateup_item(const uint16_t* __restrict__ x, int H, const void* W,
                                            const float* Ws, int inter, int hc, const int32_t* toks,
                                            int n_rows, uint16_t* __restrict__ out, uint4* xs,
                                            float* red) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int nk = H >> 6, kt0 = wave * NS;
    const char* Wb = reinterpret_cast<const char*>(W);
    uint4 wg[NS][INT8 ? 1 : 2], wu[NS][INT8 ? 1 : 2];
    tile_load<NS, INT8>(Wb + (int64_t)hc * nk * kTileBytes<INT8>, kt0, nk, lane, wg);
    tile_load<NS, INT8>(Wb + (int64_t)(inter / 16 + hc) * nk * kTileBytes<INT8>, kt0, nk, lane, wu);
    const int hc8 = H >> 3;
    for (int pass = 0; pass < n_rows; pass += kPass) {
        const int nt = min(kPass, n_rows - pass);
        __syncthreads();  // previous pass done with xs and red
        stage_x<NS>(x, H, toks, pass, nt, xs);
        __syncthreads();
#pragma unroll 1
        for (int n = 0; n < nt; ++n) {
            const uint16_t* xr = reinterpret_cast<const uint16_t*>(xs + n * hc8) + kt0 * 64 + (lane >> 4) * 16;
            float ag = 0.f, au = 0.f;
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                ag = piece_dot<INT8>(wg[s], xr + s * 64, ag);
                au = piece_dot<INT8>(wu[s], xr + s * 64, au);
            }
            ag = tile_row_sum(ag);
            au = tile_row_sum(au);
            if (lane < 16) {
                red[((wave * kPass + n) * 2) * 16 + lane] = ag;
                red[((wave * kPass + n) * 2 + 1) * 16 + lane] = au;
            }
        }
        __syncthreads();
        if (tid < nt * 16) {
            const int n = tid >> 4, r = tid & 15, col = hc * 16 + r;
            float g = 0.f, u = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                g += red[((w * kPass + n) * 2) * 16 + r];
                u += red[((w * kPass + n) * 2 + 1) * 16 + r];
            }
            if (INT8) {
                g *= Ws[col];
                u *= Ws[inter + col];
            }
            out[(int64_t)(pass + n) * inter + col] = f32_to_bf16(gelu_tanh(g) * u);
        }
    }
}

// Sum over each 32-lane half of a wavefront through DPP (no LDS): the half's
// total lands in lane 31 (lanes 0..31) and lane 63 (lanes 32..63).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float x) {
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf, false));
}
__device__ __forceinline__ float half_wave_sum_dpp(float v) {
    v = dpp_add<0x111, 0xf>(v);  // row_shr:1
    v = dpp_add<0x112, 0xf>(v);  // row_shr:2
    v = dpp_add<0x114, 0xf>(v);  // row_shr:4
    v = dpp_add<0x118, 0xf>(v);  // row_shr:8
    return dpp_add<0x142, 0xa>(v);  // row_bcast:15: row 0 into row 1, row 2 into row 3
}

// Router logits of experts [e0, e0 + 8) for tokens t0 .. t0 + nt (nt <=
// kPass): two experts per wavefront (one per half).
// logit = (sum_h x*s*W) * rms(x)^-1 * H^-0.5 + bias, all fp32; s*W is formed
// once per lane (exact products of two bf16 values), the tokens are dotted
// together, and wavefront n forms the sum of squares of token n from the
// staged x. x is requested first, so that it lands in LDS while the weights
// are in flight.
template <int NJ>
__device__ __forceinline__ void router_item(const uint16_t* __restrict__ x, int H, const uint16_t* __restrict__ scale,
                            const uint16_t* __restrict__ wr, const float* __restrict__ bias, int E,
                            int t0, int nt, float eps, float inv_sqrt_h, int e0,
                            float* __restrict__ logits, uint4* xs, float* s_rn) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int half = lane >> 5, hl = lane & 31;
    const int e = e0 + wave * 2 + half;
    const bool live = e < E;
    const int hc8 = H >> 3;
    constexpr int kPer = (kPass * 32 * NJ + kThreads - 1) / kThreads;
    uint4 xv[kPer];
    rows_load<kPer>(x, H, 0, hc8, nullptr, t0, nt * hc8, xv);
    float sw[NJ][8];
    {
        uint4 wv[NJ], sv[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int c = hl + 32 * j;
            wv[j] = reinterpret_cast<const uint4*>(wr + (int64_t)(live ? e : 0) * H)[c];
            sv[j] = reinterpret_cast<const uint4*>(scale)[c];
        }
        rows_store<kPer>(xv, nt * hc8, xs);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            float fw[8], fs[8];
            unpack8(wv[j], fw);
            unpack8(sv[j], fs);
#pragma unroll
            for (int i = 0; i < 8; ++i) sw[j][i] = fw[i] * fs[i];
        }
    }
    const float b = (live && bias) ? bias[e] : 0.f;
    __syncthreads();
    if (wave < nt) {  // rms of token t0 + wave
        float ss = 0.f;
        for (int c = lane; c < hc8; c += kWave) {
            float xf[8];
            unpack8(xs[wave * hc8 + c], xf);
#pragma unroll
            for (int i = 0; i < 8; ++i) ss += xf[i] * xf[i];
        }
        ss = wave_sum_f32(ss);
        if (lane == 0) s_rn[wave] = 1.0f / sqrtf(ss / (float)H + eps);
    }
    float acc[kPass];
#pragma unroll
    for (int n = 0; n < kPass; ++n) acc[n] = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
#pragma unroll
        for (int n = 0; n < kPass; ++n) {
            float xf[8];
            unpack8(xs[n * hc8 + hl + 32 * j], xf);  // rows n >= nt hold stale data, never stored
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[n] += sw[j][i] * xf[i];
        }
    }
#pragma unroll
    for (int n = 0; n < kPass; ++n) acc[n] = half_wave_sum_dpp(acc[n]);
    __syncthreads();  // s_rn
    if (live && hl == 31) {
#pragma unroll
        for (int n = 0; n < kPass; ++n)
            if (n < nt) logits[(int64_t)(t0 + n) * E + e] = acc[n] * (s_rn[n] * inv_sqrt_h) + b;
    }
}

// Dense gate/up partial sums, K split over kDenseSplit workgroups. Workgroup
// (hc, ks) takes K-steps [kb, kb + 4 NS), kb = 4 NS ks, of gate tile hc and
// up tile Id / 16 + hc of the tiled [2 Id, H] matrix; wavefront w takes NS of
// them from kb + w NS (steps past the matrix contribute 0). The four
// wavefronts' fp32 sums, added in wavefront order, go to
// part[ks][t][16 hc + r] (gate) and part[ks][t][Id + 16 hc + r] (up).
// The first pass's x slice is requested before the weights: loads complete in
// issue order, so it lands in LDS while the weights are still in flight.
template <int NS>
__device__ __forceinline__ void dense_gateup_part(const uint16_t* __restrict__ x, int H, const void* W,
                                                  int Id, int hc, int ks, int T,
                                                  float* __restrict__ part, uint4* xs, float* red) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int nk = H >> 6;
    const int kb = ks * kWaves * NS, kt0 = kb + wave * NS;
    const int n_steps = max(0, min(NS, nk - kt0));
    const int blk_steps = max(0, min(kWaves * NS, nk - kb));
    const char* Wb = reinterpret_cast<const char*>(W);
    const int len8 = blk_steps * 8;  // 16-byte chunks of x per token
    constexpr int kPer = (kDensePass * kWaves * NS * 8 + kThreads - 1) / kThreads;
    uint4 wg[NS][2], wu[NS][2];
    for (int pass = 0; pass < T; pass += kDensePass) {
        const int nt = min(kDensePass, T - pass);
        if (blk_steps > 0) {
            uint4 xv[kPer];
            rows_load<kPer>(x, H, kb * 64, len8, nullptr, pass, nt * len8, xv);
            if (pass == 0)
                tile_load2<NS, false>(Wb + (int64_t)hc * nk * kTileBytes<false>,
                                      Wb + (int64_t)(Id / 16 + hc) * nk * kTileBytes<false>, kt0, nk, lane, wg, wu);
            else
                __syncthreads();  // previous pass done with xs and red
            rows_store<kPer>(xv, nt * len8, xs);
            __syncthreads();
            const uint16_t* xr = reinterpret_cast<const uint16_t*>(xs) + (kt0 - kb) * 64 + (lane >> 4) * 16;
            float ag[kDensePass], au[kDensePass];
#pragma unroll
            for (int n = 0; n < kDensePass; ++n) ag[n] = au[n] = 0.f;
#pragma unroll
            for (int s = 0; s < NS; ++s)
                if (s < n_steps) {
#pragma unroll
                    for (int n = 0; n < kDensePass; ++n)
                        if (n < nt) {
                            ag[n] = piece_dot<false>(wg[s], xr + n * len8 * 8 + s * 64, ag[n]);
                            au[n] = piece_dot<false>(wu[s], xr + n * len8 * 8 + s * 64, au[n]);
                        }
                }
#pragma unroll
            for (int n = 0; n < kDensePass; ++n)
                if (n < nt) {
                    ag[n] = tile_row_sum(ag[n]);
                    au[n] = tile_row_sum(au[n]);
                    if (lane < 16) {
                        red[((wave * kDensePass + n) * 2) * 16 + lane] = ag[n];
                        red[((wave * kDensePass + n) * 2 + 1) * 16 + lane] = au[n];
                    }
                }
            __syncthreads();
        }
        if (tid < nt * 32) {
            const int n = tid >> 5, m = (tid >> 4) & 1, r = tid & 15;
            float v = 0.f;
            if (blk_steps > 0) {
#pragma unroll
                for (int w = 0; w < kWaves; ++w) v += red[((w * kDensePass + n) * 2 + m) * 16 + r];
            }
            part[((int64_t)ks * T + pass + n) * 2 * Id + m * Id + hc * 16 + r] = v;
        }
    }
}

// ---------------------------------------------------------------- K1
template <int NJ>
__global__ __launch_bounds__(kThreads) void decode_front_kernel(StreamArgs a, const uint16_t* scale,
                                                               const uint16_t* wr, const float* bias,
                                                               float eps, float inv_sqrt_h,
                                                               float* logits) {
    extern __shared__ uint4 xs[];
    // router items: (group of 8 experts) x (pass of kPass tokens)
    const int n_groups = (a.E + kRouterExperts - 1) / kRouterExperts;
    const int n_pass = (a.T + kPass - 1) / kPass;
    const int n_router = n_groups * n_pass;
    const int b = blockIdx.x;
    if (b < n_router) {
        __shared__ float s_rn[kPass];
        const int g = b % n_groups, tp = b / n_groups;
        router_item<NJ>(a.x, a.H, scale, wr, bias, a.E, tp * kPass, min(kPass, a.T - tp * kPass), eps,
                        inv_sqrt_h, g * kRouterExperts, logits, xs, s_rn);
    } else {
        // dense items: kDenseSplit K ranges of each gate/up tile pair
        __shared__ float red[kWaves * kDensePass * 2 * 16];
        const int i = b - n_router, hc = i / kDenseSplit, ks = i - hc * kDenseSplit;
        dense_gateup_part<(NJ + kDenseSplit - 1) / kDenseSplit>(a.x, a.H, a.dgu, a.Id, hc, ks, a.T,
                                                                a.dgu_part, xs, red);
    }
}

// ---------------------------------------------------------------- K3
template <int NJ, bool INT8>
__global__ __launch_bounds__(kThreads) void decode_experts_gateup_kernel(StreamArgs a) {
    extern __shared__ uint4 xs[];
    __shared__ float red[kWaves * kPass * 2 * 16];
    const int ipe = a.I / 16;  // items (16 h columns) per expert
    const int slot = blockIdx.x / ipe, hc = blockIdx.x - slot * ipe;
    if (slot >= *a.n_active) return;
    const int e = a.active[slot];
    const int p0 = a.offsets[e], n = a.offsets[e + 1] - p0;
    const int64_t wstride = (int64_t)2 * a.I * a.H;
    const void* W = INT8 ? (const void*)((const int8_t*)a.gu + e * wstride)
                         : (const void*)((const uint16_t*)a.gu + e * wstride);
    const float* Ws = INT8 ? a.gu_scale + (int64_t)e * 2 * a.I : nullptr;
    gateup_item<NJ, INT8>(a.x, a.H, W, Ws, a.I, hc, a.perm_token + p0, n, a.h + (int64_t)p0 * a.I,
                          xs, red);
}

// ---------------------------------------------------------------- K2
// Dense gate/up finish: hd[t][c] = gelu_tanh(gate) * up, each the sum of its
// kDenseSplit partial sums in split order; one thread per (t, c).
__device__ __forceinline__ void dense_finish(const StreamArgs& a, int blk) {
    const int i = blk * kRouteThreads + threadIdx.x;
    if (i >= a.T * a.Id) return;
    const int t = i / a.Id, c = i - t * a.Id;
    float gp[kDenseSplit], up[kDenseSplit];
#pragma unroll
    for (int ks = 0; ks < kDenseSplit; ++ks) {
        const float* row = a.dgu_part + ((int64_t)ks * a.T + t) * 2 * a.Id;
        gp[ks] = row[c];
        up[ks] = row[a.Id + c];
    }
    float g = gp[0], u = up[0];
#pragma unroll
    for (int ks = 1; ks < kDenseSplit; ++ks) {
        g += gp[ks];
        u += up[ks];
    }
    a.hd[(int64_t)t * a.Id + c] = f32_to_bf16(gelu_tanh(g) * u);
}

// Workgroup 0 routes every token (ONNX export card, "Truthful graph
// contracts", row "Router"), the other workgroups finish the dense gate/up.
//
// Selection by rank, one thread per (token, expert) pair: each logit becomes
// the 64-bit composite (order-preserving key, ~expert), so that a larger
// composite means a larger logit or, for equal logits, the lower expert; the
// rank of a pair is the number of its token's composites above its own, and
// ranks 0 .. K-1 are the top K in order (descending logit, ties to the lower
// index). The renormalised weight of the k-th selected expert is
// exp(l_k - l_0) / sum_j exp(l_j - l_0) over the K selected (the softmax
// denominator over all experts cancels in the renormalisation), summed in k
// order, times its per-expert scale.
//
// Then the stable grouping by expert. With T <= 64 every token is one bit of a
// 64-bit mask per expert: the rank of pair (t, k) within its expert is the
// number of lower tokens in that expert's mask, the expert's row count its
// popcount.
__global__ __launch_bounds__(kRouteThreads) void decode_route_kernel(StreamArgs a, const float* logits,
                                                                    const float* pes,
                                                                    int32_t* topk_idx, float* topk_w) {
    if (!logits || blockIdx.x > 0) {
        dense_finish(a, (int)blockIdx.x - (logits ? 1 : 0));
        return;
    }
    __shared__ int s_idx[kMaxPairs];
    __shared__ float s_w[kMaxPairs];
    __shared__ float s_l[kMaxPairs];   // logit of each selected pair
    __shared__ float s_e[kMaxPairs];   // its exp relative to the token's largest
    __shared__ unsigned long long s_mask[kMaxExperts];
    __shared__ int s_off[kMaxExperts + 1];
    __shared__ float s_pes[kMaxExperts];
    __shared__ unsigned long long s_comp[kRouteThreads];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int T = a.T, K = a.K, E = a.E, TK = T * K;
    // experts padded to a power of two: a chunk holds kRouteThreads / Ep tokens
    const int Ep = E <= 64 ? 64 : E <= 128 ? 128 : 256;
    const int tc = kRouteThreads / Ep;
    const int tl = tid / Ep, e = tid - tl * Ep;
    if (tid < E) {
        s_mask[tid] = 0ull;
        s_pes[tid] = pes[tid];
    }
    for (int t0 = 0; t0 < T; t0 += tc) {
        const int t = t0 + tl;
        const bool live = t < T && e < E;
        const float l = live ? logits[(int64_t)t * E + e] : 0.f;
        const unsigned long long comp =
            live ? ((unsigned long long)order_key(l) << 32) | (unsigned)(~e) : 0ull;
        if (t0 > 0) __syncthreads();  // previous chunk done with s_comp
        s_comp[tid] = comp;
        __syncthreads();
        if (live) {
            const unsigned long long* row = s_comp + tl * Ep;
            int rank = 0;
            for (int j = 0; j < E; j += 2) {  // an odd E reads the padding slot E, which holds 0
                const unsigned long long c0 = row[j], c1 = row[j + 1];
                rank += (c0 > comp) + (c1 > comp);
            }
            if (rank < K) {
                s_idx[t * K + rank] = e;
                s_l[t * K + rank] = l;
            }
        }
    }
    __syncthreads();
    if (tid < TK)  // exp of each selected logit relative to the token's largest
        s_e[tid] = expf(s_l[tid] - s_l[(tid / K) * K]);
    __syncthreads();
    if (tid < TK) {
        const int t = tid / K;
        float sum = 0.f;
        for (int k = 0; k < K; ++k) sum += s_e[t * K + k];
        const int ei = s_idx[tid];
        const float wt = s_e[tid] / sum * s_pes[ei];
        s_w[tid] = wt;
        topk_idx[tid] = ei;
        topk_w[tid] = wt;
    }
    __syncthreads();
    if (tid < TK) atomicOr(&s_mask[s_idx[tid]], 1ull << (tid / K));
    __syncthreads();
    if (wave == 0) {
        int c[4], act[4], csum = 0, asum = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = lane * 4 + i;
            c[i] = e < E ? __popcll(s_mask[e]) : 0;
            act[i] = c[i] > 0;
            csum += c[i];
            asum += act[i];
        }
        int ci = csum, ai = asum;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int u = __shfl_up(ci, off, kWave), v = __shfl_up(ai, off, kWave);
            if (lane >= off) {
                ci += u;
                ai += v;
            }
        }
        int crun = ci - csum, arun = ai - asum;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = lane * 4 + i;
            if (e < E) {
                s_off[e] = crun;
                a.offsets[e] = crun;
                a.counts[e] = c[i];
                if (act[i]) a.active[arun] = e;
            }
            crun += c[i];
            arun += act[i];
        }
        if (lane == kWave - 1) {
            a.offsets[E] = ci;
            *a.n_active = ai;
        }
    }
    __syncthreads();
    if (tid < TK) {
        const int e = s_idx[tid], t = tid / K;
        const int pos = s_off[e] + __popcll(s_mask[e] & ((1ull << t) - 1ull));
        a.perm_token[pos] = t;
        a.perm_w[pos] = s_w[tid];
        a.inv_row[tid] = pos;
    }
}

// ---------------------------------------------------------------- K4
// Down projections. A wavefront reads K-steps [kt0, kt0 + n_steps) (n_steps <=
// NS) of one 16-row tile of a tiled [H, inter] matrix and dots them with the
// token rows of h (or hd) staged in LDS; returns, in lanes 0..15, the partial
// sum of row lane of the tile for token n of the pass.
template <int NS, bool INT8>
__device__ __forceinline__ float down_dot(const uint4 (&w)[NS][INT8 ? 1 : 2], const uint16_t* hrow,
                                          int kt0, int n_steps, int lane) {
    const uint16_t* hp = hrow + kt0 * 64 + (lane >> 4) * 16;
    float acc = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s)
        if (s < n_steps) acc = piece_dot<INT8>(w[s], hp + s * 64, acc);
    return tile_row_sum(acc);
}

template <int NS, bool INT8>
__global__ __launch_bounds__(kThreads) void decode_down_kernel(StreamArgs a) {
    extern __shared__ uint4 hs[];  // [kPass][max(I, Id)] bf16
    __shared__ float red[kWaves * kPass * 16];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int ipe = a.H / 64;  // expert items: 4 tiles (one per wavefront) of 16 rows
    // the dense items (a longer reduction each) come first in the grid, so
    // that they run beside the expert items instead of after them
    const int dense_items = a.with_dense ? a.H / 16 : 0;
    const int b = (int)blockIdx.x - dense_items;
    if (b >= 0) {
        const int slot = b / ipe, g = b - slot * ipe;
        if (slot >= *a.n_active) return;
        const int e = a.active[slot];
        const int p0 = a.offsets[e], n_rows = a.offsets[e + 1] - p0;
        const int64_t wstride = (int64_t)a.H * a.I;
        const char* W = INT8 ? (const char*)((const int8_t*)a.dw + e * wstride)
                             : (const char*)((const uint16_t*)a.dw + e * wstride);
        const int nk = a.I >> 6, tile = g * kWaves + wave;
        uint4 w[NS][INT8 ? 1 : 2];
        tile_load<NS, INT8>(W + (int64_t)tile * nk * kTileBytes<INT8>, 0, nk, lane, w);
        const float sc = INT8 ? a.dw_scale[(int64_t)e * a.H + tile * 16 + (lane & 15)] : 1.f;
        const int hc8 = a.I >> 3;
        for (int pass = 0; pass < n_rows; pass += kPass) {
            const int nt = min(kPass, n_rows - pass);
            __syncthreads();
            stage_rows<(kPass * 128 + kThreads - 1) / kThreads>(
                reinterpret_cast<const uint4*>(a.h + (int64_t)(p0 + pass) * a.I), nt * hc8, hs);
            __syncthreads();
#pragma unroll 1
            for (int n = 0; n < nt; ++n) {
                const float v = down_dot<NS, INT8>(w, reinterpret_cast<const uint16_t*>(hs + n * hc8), 0,
                                                   nk, lane);
                if (lane < 16) a.part[(int64_t)(p0 + pass + n) * a.H + tile * 16 + lane] = v * sc;
            }
        }
    } else {
        // dense down: one 16-row tile per workgroup, K split over the wavefronts
        const int tile = (int)blockIdx.x;
        const int nk = a.Id >> 6, kd = (nk + kWaves - 1) / kWaves;
        const int kt0 = wave * kd, n_steps = max(0, min(kd, nk - kt0));
        uint4 w[NS][2];
        tile_load<NS, false>(reinterpret_cast<const char*>(a.ddw) + (int64_t)tile * nk * kTileBytes<false>,
                             kt0, nk, lane, w);
        const int hc8 = a.Id >> 3;
        for (int pass = 0; pass < a.T; pass += kPass) {
            const int nt = min(kPass, a.T - pass);
            __syncthreads();
            stage_rows<(kPass * 512 + kThreads - 1) / kThreads>(
                reinterpret_cast<const uint4*>(a.hd + (int64_t)pass * a.Id), nt * hc8, hs);
            __syncthreads();
#pragma unroll 1
            for (int n = 0; n < nt; ++n) {
                const float v = down_dot<NS, false>(w, reinterpret_cast<const uint16_t*>(hs + n * hc8),
                                                    kt0, n_steps, lane);
                if (lane < 16) red[(wave * kPass + n) * 16 + lane] = v;
            }
            __syncthreads();
            if (tid < nt * 16) {
                const int n = tid >> 4, r = tid & 15;
                float v = 0.f;
#pragma unroll
                for (int ww = 0; ww < kWaves; ++ww) v += red[(ww * kPass + n) * 16 + r];
                a.dpart[(int64_t)(pass + n) * a.H + tile * 16 + r] = v;
            }
        }
    }
}

// ---------------------------------------------------------------- K5
// y[t] = dense[t] + sum_k w[t,k] * expert rows, in k order (row "MoE topology").
__global__ __launch_bounds__(kThreads) void decode_combine_kernel(StreamArgs a) {
    const int i = blockIdx.x * kThreads + threadIdx.x;  // one thread per 4 features
    const int per_row = a.H / 4;
    if (i >= a.T * per_row) return;
    const int t = i / per_row, c = (i - t * per_row) * 4;
    float4 v = *reinterpret_cast<const float4*>(a.dpart + (int64_t)t * a.H + c);
    if (a.max_active > 0) {
        int p[kMaxTopK];
#pragma unroll
        for (int k = 0; k < kMaxTopK; ++k) p[k] = a.inv_row[(int64_t)t * a.K + min(k, a.K - 1)];
        float wk[kMaxTopK];
        float4 r[kMaxTopK];
#pragma unroll
        for (int k = 0; k < kMaxTopK; ++k) {
            wk[k] = a.perm_w[p[k]];
            r[k] = *reinterpret_cast<const float4*>(a.part + (int64_t)p[k] * a.H + c);
        }
#pragma unroll
        for (int k = 0; k < kMaxTopK; ++k) {
            if (k < a.K) {
                v.x += wk[k] * r[k].x;
                v.y += wk[k] * r[k].y;
                v.z += wk[k] * r[k].z;
                v.w += wk[k] * r[k].w;
            }
        }
    }
    *reinterpret_cast<uint2*>(a.y + (int64_t)t * a.H + c) =
        make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
}

template <int NJ>
hipError_t launch_front_nj(const StreamArgs& a, const uint16_t* scale, const uint16_t* wr,
                           const float* bias, float eps, float* logits, bool router,
                           hipStream_t stream) {
    const int n_router =
        router ? ((a.E + kRouterExperts - 1) / kRouterExperts) * ((a.T + kPass - 1) / kPass) : 0;
    const int blocks = n_router + (a.with_dense ? (a.Id / 16) * kDenseSplit : 0);
    // x rows of a router pass, or the x slices of a dense pass
    const int ns = (a.H / 256 + kDenseSplit - 1) / kDenseSplit;
    const size_t lds = (size_t)max(kPass * a.H, kDensePass * kWaves * ns * 64) * sizeof(uint16_t);
    const float inv_sqrt_h = (float)(1.0 / __builtin_sqrt((double)a.H));
    if (blocks <= 0) return hipSuccess;
    StreamArgs b = a;
    if (!router) b.E = 0;  // no router items: the kernel derives their count from E
    hipLaunchKernelGGL(decode_front_kernel<NJ>, dim3(blocks), dim3(kThreads), lds, stream, b, scale,
                       wr, bias, eps, inv_sqrt_h, logits);
    return hipGetLastError();
}

template <int NJ>
hipError_t launch_experts_nj(const StreamArgs& a, bool int8, hipStream_t stream) {
    const int blocks = a.max_active * (a.I / 16);
    const size_t lds = (size_t)kPass * a.H * sizeof(uint16_t);
    if (int8)
        hipLaunchKernelGGL((decode_experts_gateup_kernel<NJ, true>), dim3(blocks), dim3(kThreads), lds, stream, a);
    else
        hipLaunchKernelGGL((decode_experts_gateup_kernel<NJ, false>), dim3(blocks), dim3(kThreads), lds, stream, a);
    return hipGetLastError();
}

}  // namespace

// NJ = H / 256 K-steps per wavefront; instantiated for hidden sizes up to 3072.
#define MOE_NJ_SWITCH(nj, CALL)                                   \
    switch (nj) {                                                 \
        case 1: return CALL(1);   case 2: return CALL(2);         \
        case 3: return CALL(3);   case 4: return CALL(4);         \
        case 5: return CALL(5);   case 6: return CALL(6);         \
        case 7: return CALL(7);   case 8: return CALL(8);         \
        case 9: return CALL(9);   case 10: return CALL(10);       \
        case 11: return CALL(11); case 12: return CALL(12);       \
        default: return hipErrorInvalidValue;                     \
    }

hipError_t launch_decode_front(const StreamArgs& a, const uint16_t* scale, const uint16_t* wr,
                               const float* bias, float eps, float* logits, hipStream_t stream) {
#define CALL(n) launch_front_nj<n>(a, scale, wr, bias, eps, logits, logits != nullptr, stream)
    MOE_NJ_SWITCH(a.H / 256, CALL)
#undef CALL
}

hipError_t launch_decode_route(const StreamArgs& a, const float* logits, const float* pes,
                               int32_t* topk_idx, float* topk_w, hipStream_t stream) {
    const int blocks =
        (logits ? 1 : 0) + (a.with_dense ? (a.T * a.Id + kRouteThreads - 1) / kRouteThreads : 0);
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(decode_route_kernel, dim3(blocks), dim3(kRouteThreads), 0, stream, a, logits, pes,
                       topk_idx, topk_w);
    return hipGetLastError();
}

hipError_t launch_decode_experts_gateup(const StreamArgs& a, bool int8, hipStream_t stream) {
#define CALL(n) launch_experts_nj<n>(a, int8, stream)
    MOE_NJ_SWITCH(a.H / 256, CALL)
#undef CALL
}

hipError_t launch_decode_down(const StreamArgs& a, bool int8, hipStream_t stream) {
    // K-steps a wavefront holds: a whole expert tile (I / 64) or a quarter of
    // a dense tile (Id / 256, rounded up)
    const int need = max(a.I / 64, (a.Id / 64 + kWaves - 1) / kWaves);
    const int blocks = a.max_active * (a.H / 64) + (a.with_dense ? a.H / 16 : 0);
    if (blocks <= 0) return hipSuccess;
    const size_t lds = (size_t)kPass * (a.I > a.Id ? a.I : a.Id) * sizeof(uint16_t);
    const dim3 grid(blocks), block(kThreads);
#define LAUNCH(N)                                                                                   \
    do {                                                                                            \
        if (int8) hipLaunchKernelGGL((decode_down_kernel<N, true>), grid, block, lds, stream, a);   \
        else hipLaunchKernelGGL((decode_down_kernel<N, false>), grid, block, lds, stream, a);       \
        return hipGetLastError();                                                                   \
    } while (0)
    if (need <= 2) LAUNCH(2);
    if (need <= 4) LAUNCH(4);
    if (need <= 8) LAUNCH(8);
    if (need <= 11) LAUNCH(11);
    if (need <= 12) LAUNCH(12);
    if (need <= 16) LAUNCH(16);
#undef LAUNCH
    return hipErrorInvalidValue;
}

hipError_t launch_decode_combine(const StreamArgs& a, hipStream_t stream) {
    const int n = a.T * (a.H / 4);
    hipLaunchKernelGGL(decode_combine_kernel, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace moe
