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
//   K1 decode_front: router partial logits (16 experts per workgroup), as
//      bf16 MFMAs of the batch against 16-row weight tiles, the K range split
//      over kFrontSplit workgroups (fp32 partial sums). (The dense MLP alone
//      runs its gate/up items here too.)
//   K2 decode_route: one workgroup: the logits from the partial sums, the
//      softmax/top-k of every token (ONNX export card, "Truthful graph
//      contracts", row "Router") and the grouping of the routed pairs by
//      expert (counts, offsets, grouped rows, inverse rows, list of touched
//      experts); beside it, the dense MLP's gate/up tiles (fp32 partial sums,
//      as in K1), which only need x: K1 then holds the router alone.
//   K3 decode_experts_gateup: half the K range of 16 gate columns (+ the 16
//      matching up columns) of one touched expert per workgroup, split over
//      its 4 wavefronts; every weight byte is read exactly once with wide
//      non-temporal loads issued before anything waits, then dotted with the
//      expert's tokens staged in LDS. fp32 partial sums per half; K4 adds the
//      halves and forms h = gelu_tanh(gate) * up when it stages h. Its first
//      workgroups add the dense gate/up partial sums and form the dense
//      intermediate gelu_tanh(gate) * up.
//   K4 decode_down: one 16-row tile of a touched expert's down matrix per
//      wavefront (fp32 partial rows per routed pair), and the dense down
//      matrix with K split over a workgroup's wavefronts.
//   K5 decode_combine: y = dense + sum_k w_k * expert_k in k order (row "MoE
//      topology"), without atomics.
// int8 experts (int8 experts card, "How it works") are read as int8, widened
// exactly in registers, and their per-row scale multiplies the dot product.
// E4M3 experts (the vLLM recipe's fp8 variant) are widened to half carriers by
// bit placement and dotted with x quantised per token (decode_front's last
// workgroups); h is formed and quantised per routed row by decode_hquant.
// The template parameter WQ names the experts' format: 0 bf16, 1 int8, 2 E4M3.
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "topk.h"
#include "../../include/moe.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kPass = 4;           // tokens staged per pass
constexpr int kRouteThreads = 1024;
constexpr int kMaxPairs = MOE_STREAM_MAX_TOKENS * MOE_MAX_TOPK;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld_nt16(const void* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
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

// Four per-row values of a pass (rows past nt repeat row nt - 1), as four
// uniform scalars: pick(r) is a chain of selects, never an indexed array or a
// load through a selected address (readfirstlane keeps the compiler from
// folding the selects into the loads).
template <class T>
struct QuadOf {
    T v0, v1, v2, v3;
    __device__ __forceinline__ T pick(int r) const { return r == 3 ? v3 : r == 2 ? v2 : r == 1 ? v1 : v0; }
    __device__ __forceinline__ static T uni(T v) {
        return __builtin_bit_cast(T, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
    }
    __device__ __forceinline__ static QuadOf load(const T* __restrict__ p, int nt) {
        return {uni(p[0]), uni(p[min(1, nt - 1)]), uni(p[min(2, nt - 1)]), uni(p[min(3, nt - 1)])};
    }
};
typedef QuadOf<int32_t> Quad;

typedef __attribute__((address_space(3))) void lds_void_t;

// The activations a workgroup stages (x rows, h partial sums, h rows) go
// straight from global memory into LDS (buffer_load_dwordx4 ... lds): no
// registers hold them and nothing waits for them until the caller's dma_wait,
// so they are issued right behind the weights and land right behind them.
// Chunk j (16 bytes) of n is read at byte offset off(j) of a buffer of `bytes`
// bytes from `base` (reads past it return zero) and lands at dst[j];
// wavefront w's load q moves chunks (q kWaves + w) 64 .. + 64. Every
// wavefront issues all KQ loads (a load under a branch makes the compiler's
// wait counts after the join wait for every load in flight, the weights
// included); chunks past n fetch chunk n - 1, so the caller reserves KQ kWaves
// 64 chunks of LDS from dst. (A buffer load, unlike global_load_lds, leaves
// the compiler's counts for the weights' own waits exact.) The compiler must
// not move loads across these (the waits count loads in issue order), nor
// schedule work on the loads in flight ahead of them: compiler memory and
// scheduling barriers on both sides.
template <int KQ, class Off>
__device__ __forceinline__ void dma_chunks(uint4* dst, int n, const void* base, int64_t bytes, Off off) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)min(bytes, (int64_t)INT32_MAX),
                                          0x00020000);  // raw 32-bit data format
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6), lane = threadIdx.x & 63;
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < KQ; ++q) {
        const int b = (q * kWaves + wave) * 64;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(dst + b), 16, (int)off(min(b + lane, n - 1)), 0, 0,
                                                 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
}
// Every load of the wavefront done (its DMA chunks in LDS); a barrier then
// makes all wavefronts' chunks visible.
__device__ __forceinline__ void dma_wait() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// 16 int8 (one tiled-layout piece) -> two groups of 8 bf16 (exact)
__device__ __forceinline__ void i8x16_to_bf16(const uint4& v, uint4& lo, uint4& hi) {
    lo = i8x8_to_bf16(make_uint4(v.x, v.y, 0u, 0u));
    hi = i8x8_to_bf16(make_uint4(v.z, v.w, 0u, 0u));
}
// 16 E4M3 codes (one tiled-layout piece) -> two groups of 8 half carriers (value * 2^-8, exact)
__device__ __forceinline__ void f8x16_to_f16(const uint4& v, uint4& lo, uint4& hi) {
    lo = make_uint4(fp8pair_to_f16(v.x, 0), fp8pair_to_f16(v.x, 16), fp8pair_to_f16(v.y, 0),
                    fp8pair_to_f16(v.y, 16));
    hi = make_uint4(fp8pair_to_f16(v.z, 0), fp8pair_to_f16(v.z, 16), fp8pair_to_f16(v.w, 0),
                    fp8pair_to_f16(v.w, 16));
}
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
// acc + a.lo*b.lo + a.hi*b.hi on packed halves (v_dot2_f32_f16: the products of
// two half carriers of E4M3 values are exact in fp32)
__device__ __forceinline__ float dot8_f16(const uint4& a, const uint4& b, float acc) {
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a.x), __builtin_bit_cast(f16x2_t, b.x), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a.y), __builtin_bit_cast(f16x2_t, b.y), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a.z), __builtin_bit_cast(f16x2_t, b.z), acc, false);
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a.w), __builtin_bit_cast(f16x2_t, b.w), acc, false);
}

// 1-byte weights are widened ahead of their use: a lane's piece of a K-step
// (16 k in one 16-byte load) becomes two groups of 8 bf16 (int8, exact) or
// half carriers (E4M3), the layout of a bf16 piece (two 16-byte halves, 8 k
// each), and its dot product with the 16 matching x values (for E4M3 the half
// carriers of x) needs no further conversion.
template <int WQ>
__device__ __forceinline__ void widen_piece(const uint4& v, uint4 (&o)[2]) {
    if (WQ == 2) f8x16_to_f16(v, o[0], o[1]);
    else i8x16_to_bf16(v, o[0], o[1]);
}
// one K-step of a lane's bf16 (or widened) piece dotted with the 16 matching x values
template <int WQ>
__device__ __forceinline__ float wide_dot(const uint4 (&w)[2], const uint16_t* xp, float acc) {
    const uint4 x0 = *reinterpret_cast<const uint4*>(xp);
    const uint4 x1 = *reinterpret_cast<const uint4*>(xp + 8);
    if (WQ == 2) return dot8_f16(w[1], x1, dot8_f16(w[0], x0, acc));
    return dot8_bf16(w[1], x1, dot8_bf16(w[0], x0, acc));
}
// Widens every step's piece as soon as it lands, in load order. The pin
// before each piece keeps its conversion after the activations' copies issued
// ahead of it (the scheduler would otherwise start converting, and so wait for
// the weights, before issuing them); the pin after it keeps the compiler from
// sinking the conversion to its first use (after the activations are staged).
// The conversion then overlaps the weights still in flight instead of
// following the last of them.
template <int NS, int WQ>
__device__ __forceinline__ void widen_steps(uint4 (&w)[NS][1], uint4 (&o)[NS][2]) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        u32x4 v{w[s][0].x, w[s][0].y, w[s][0].z, w[s][0].w};  // one 128-bit operand: no copies
        asm volatile("" : "+v"(v));
        widen_piece<WQ>(make_uint4(v.x, v.y, v.z, v.w), o[s]);
        asm volatile("" : "+v"(o[s][0].x), "+v"(o[s][0].y), "+v"(o[s][0].z), "+v"(o[s][0].w),
                     "+v"(o[s][1].x), "+v"(o[s][1].y), "+v"(o[s][1].z), "+v"(o[s][1].w));
    }
}

// sum of the four lanes holding one row of a tile (lanes r, r+16, r+32, r+48)
__device__ __forceinline__ float tile_row_sum(float v) {
    v += __shfl_xor(v, 16, kWave);
    return v + __shfl_xor(v, 32, kWave);
}

template <int WQ>
constexpr int kTileBytes = WQ ? 1024 : 2048;

// Load steps kt0 .. kt0 + NS - 1 (clamped to the last step nk - 1) of this
// lane's pieces of a tile whose step 0 starts at `tile`; all loads issued at once.
template <int NS, int WQ>
__device__ __forceinline__ void tile_load(const char* tile, int kt0, int nk, int lane,
                                          uint4 (&w)[NS][WQ ? 1 : 2]) {
    const char* p = tile + lane * 16;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int64_t off = (int64_t)min(kt0 + s, nk - 1) * kTileBytes<WQ>;
        w[s][0] = ld_nt16(p + off);
        if (!WQ) w[s][WQ ? 0 : 1] = ld_nt16(p + off + 1024);
    }
}

// tile_load of two tiles at once, their loads interleaved step by step (so
// that step s of both has landed once 2 (s + 1) of them have).
template <int NS, int WQ>
__device__ __forceinline__ void tile_load2(const char* ta, const char* tb, int kt0, int nk, int lane,
                                           uint4 (&wa)[NS][WQ ? 1 : 2], uint4 (&wb)[NS][WQ ? 1 : 2]) {
    const char* pa = ta + lane * 16;
    const char* pb = tb + lane * 16;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int64_t off = (int64_t)min(kt0 + s, nk - 1) * kTileBytes<WQ>;
        wa[s][0] = ld_nt16(pa + off);
        if (!WQ) wa[s][WQ ? 0 : 1] = ld_nt16(pa + off + 1024);
        wb[s][0] = ld_nt16(pb + off);
        if (!WQ) wb[s][WQ ? 0 : 1] = ld_nt16(pb + off + 1024);
    }
}

// Half `half` of the K range of the gate/up of 16 h columns (gate tile hc and
// up tile inter/16 + hc) against tokens tok(0 .. n_rows): fp32 partial sums
// part[half][p][16 hc + r] (gate) and part[half][p][inter + 16 hc + r] (up),
// p the grouped row. Wavefront w takes NS of the half's K-steps from
// kb + w NS (steps past the half contribute 0); only the half's columns of x
// are staged.
template <int NS, int WQ>
__device__ __forceinline__ void gateup_half_item(const uint16_t* __restrict__ x, int64_t x_bytes, int H, const void* W,
                                                 int inter,
                                                 int hc, int half, const int32_t* __restrict__ toks, int n_rows,
                                                 int64_t half_stride, float* __restrict__ part, uint4* xs,
                                                 float* red) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int nk = H >> 6, hk = nk >> 1;  // K-steps of a half
    const int kb = half * hk, kt0 = kb + wave * NS, ke = kb + hk;
    const int n_steps = max(0, min(NS, ke - kt0));
    const char* Wb = reinterpret_cast<const char*>(W);
    const int len8 = hk * 8;  // 16-byte chunks of x per token in the half
    // x rows of a pass's tokens -> LDS, chunk i of token i / len8. The token
    // indices are uniform loads (the scalar path, beside the weights' vector
    // loads), kept as four values rather than an array, which the compiler
    // would index through memory.
    static_assert(kPass == 4, "four token values a pass");
    Quad tk;
    constexpr int kXQ = (kPass * 32 * NS + kThreads - 1) / kThreads;  // DMA loads a wavefront issues
    auto stage_x = [&](int nt) {
        dma_chunks<kXQ>(xs, nt * len8, x, x_bytes, [&](int i) {
            const int r = i / len8;
            return (tk.pick(r) * H + kb * 64) * 2 + (i - r * len8) * 16;
        });
    };
    tk = Quad::load(toks, min(kPass, n_rows));
    uint4 wg[NS][WQ ? 1 : 2], wu[NS][WQ ? 1 : 2];
    // loads clamped to the half's last step
    tile_load<NS, WQ>(Wb + (int64_t)hc * nk * kTileBytes<WQ>, kt0, ke, lane, wg);
    tile_load<NS, WQ>(Wb + (int64_t)(inter / 16 + hc) * nk * kTileBytes<WQ>, kt0, ke, lane, wu);
    stage_x(min(kPass, n_rows));  // the first pass's x, right behind the weights
    // 1-byte weights: widened as they land (the gate tile's steps first, in load order)
    uint4 wgw[NS][2], wuw[NS][2];
    if constexpr (WQ != 0) {
        widen_steps<NS, WQ>(wg, wgw);
        widen_steps<NS, WQ>(wu, wuw);
    }
    for (int pass = 0; pass < n_rows; pass += kPass) {
        const int nt = min(kPass, n_rows - pass);
        if (pass > 0) {
            __syncthreads();  // previous pass done with xs and red
            tk = Quad::load(toks + pass, nt);
            stage_x(nt);
        }
        dma_wait();
        __syncthreads();
#pragma unroll 1
        for (int t = 0; t < nt; ++t) {
            const uint16_t* xr =
                reinterpret_cast<const uint16_t*>(xs + t * len8) + (kt0 - kb) * 64 + (lane >> 4) * 16;
            float ag = 0.f, au = 0.f;
#pragma unroll
            for (int st = 0; st < NS; ++st)
                if (st < n_steps) {
                    if constexpr (WQ != 0) {
                        ag = wide_dot<WQ>(wgw[st], xr + st * 64, ag);
                        au = wide_dot<WQ>(wuw[st], xr + st * 64, au);
                    } else {
                        ag = wide_dot<0>(wg[st], xr + st * 64, ag);
                        au = wide_dot<0>(wu[st], xr + st * 64, au);
                    }
                }
            ag = tile_row_sum(ag);
            au = tile_row_sum(au);
            if (lane < 16) {
                red[((wave * kPass + t) * 2) * 16 + lane] = ag;
                red[((wave * kPass + t) * 2 + 1) * 16 + lane] = au;
            }
        }
        __syncthreads();
        if (tid < nt * 32) {
            const int t = tid >> 5, m = (tid >> 4) & 1, r = tid & 15;
            float v = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) v += red[((w * kPass + t) * 2 + m) * 16 + r];
            part[half * half_stride + (int64_t)(pass + t) * 2 * inter + m * inter + hc * 16 + r] = v;
        }
    }
}

// ---------------------------------------------------------------- K1
// The front items are small matrix products of the batch (T <= 64 tokens,
// taken 16 at a time as the M rows of a bf16 MFMA 16x16x32) with 16-row weight
// tiles. The tiled layout gives lane l the 16 k values 16 (l / 16) .. + 16 of
// row l % 16 of a 64-wide K-step, which is the MFMA B operand of two MFMAs
// (its first and second 8 values) once the A operand enumerates the same k:
// lane l loads x[token l % 16][64 kt + 16 (l / 16) .. + 16] straight from
// global memory. Token rows past the batch repeat its last token and are never
// stored. The K range of an item is split over kFrontSplit workgroups of four
// wavefronts (NS K-steps each); a workgroup adds its wavefronts' sums in
// wavefront order through LDS and writes fp32 partial sums of its slice.

__device__ __forceinline__ f32x4_t mfma16(const uint4& a, const uint4& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// A fragments of K-steps kt0 .. kt0 + NS - 1 (clamped to the last step) for
// token row tok.
template <int NS>
__device__ __forceinline__ void a_frags(const uint16_t* __restrict__ x, int H, int tok, int kt0, int nk,
                                        int lane, uint4 (&a)[NS][2]) {
    const uint16_t* row = x + (int64_t)tok * H + (lane >> 4) * 16;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const uint4* p = reinterpret_cast<const uint4*>(row + min(kt0 + s, nk - 1) * 64);
        a[s][0] = p[0];
        a[s][1] = p[1];
    }
}

// The 16 x 16 accumulators of the four wavefronts (red[w][m][row][col], m <
// n_m matrices) summed in wavefront order; output o = tid + 256 q is
// (m, row, col) = (o / 256, o / 16 % 16, o % 16).
__device__ __forceinline__ void red_store(float* red, int wave, int m, int lane, const f32x4_t& c) {
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(wave * 2 + m) * 256 + ((lane >> 4) * 4 + i) * 16 + (lane & 15)] = c[i];
}
__device__ __forceinline__ float red_sum(const float* red, int m, int rc) {
    float v = red[m * 256 + rc];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) v += red[(w * 2 + m) * 256 + rc];
    return v;
}

// Dense gate/up, item (hc, ks): gate tile hc and up tile Id / 16 + hc of the
// tiled [2 Id, H] matrix over K-steps [4 NS ks, 4 NS (ks + 1)) (steps past the
// matrix contribute 0) -> part[ks][t][16 hc + c] (gate), part[ks][t][Id + 16 hc + c] (up).
// Run by a group of 256 threads (tid: the thread's index in the group); every
// thread of the workgroup takes part in its barriers.
template <int NS>
__device__ __forceinline__ void dense_gateup_part(const uint16_t* __restrict__ x, int H, const void* W, int Id,
                                                  int hc, int ks, int T, float* __restrict__ part, float* red,
                                                  int tid) {
    const int wave = tid >> 6, lane = tid & 63;
    const int nk = H >> 6;
    const int kt0 = (ks * kWaves + wave) * NS;
    const int n_steps = max(0, min(NS, nk - kt0));
    const char* Wb = reinterpret_cast<const char*>(W);
    uint4 wg[NS][2], wu[NS][2];
    for (int pass = 0; pass < T; pass += 16) {
        uint4 xa[NS][2];
        a_frags<NS>(x, H, min(pass + (lane & 15), T - 1), kt0, nk, lane, xa);
        if (pass == 0)
            tile_load2<NS, false>(Wb + (int64_t)hc * nk * kTileBytes<false>,
                                  Wb + (int64_t)(Id / 16 + hc) * nk * kTileBytes<false>, kt0, nk, lane, wg, wu);
        f32x4_t cg = {0.f, 0.f, 0.f, 0.f}, cu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NS; ++s)
            if (s < n_steps) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    cg = mfma16(xa[s][h], wg[s][h], cg);
                    cu = mfma16(xa[s][h], wu[s][h], cu);
                }
            }
        if (pass > 0) __syncthreads();  // the previous pass is done with red
        red_store(red, wave, 0, lane, cg);
        red_store(red, wave, 1, lane, cu);
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int o = tid + kThreads * q, m = o >> 8, rc = o & 255, r = rc >> 4, c = rc & 15;
            if (pass + r < T)
                part[((int64_t)ks * T + pass + r) * 2 * Id + m * Id + hc * 16 + c] = red_sum(red, m, rc);
        }
    }
}

// Router, item (nt, ks): partial logits of experts [16 nt, 16 nt + 16) over
// the same K range. The B operand is s*W of the row-major router matrix,
// split into bf16 hi and lo (exact products, fp32 accumulation); the lanes
// also add the squares of their x values, and the four lanes of a token row
// (l, l + 16, l + 32, l + 48) then the wavefronts add them up.
// -> lpart[ks][t][e] = sum over the range of x[t] * s * W[e]; ss[ks][t] = sum of x[t]^2
// (written by the items of nt = 0).
template <int NS>
__device__ __forceinline__ void router_part(const uint16_t* __restrict__ x, int H,
                                            const uint16_t* __restrict__ scale, const uint16_t* __restrict__ wr,
                                            int E, int nt, int ks, int T, float* __restrict__ lpart,
                                            float* __restrict__ ss_part, float* red) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int nk = H >> 6;
    const int kt0 = (ks * kWaves + wave) * NS;
    const int n_steps = max(0, min(NS, nk - kt0));
    const int e = min(nt * 16 + (lane & 15), E - 1);
    uint4 bh[NS][2], bl[NS][2];
    {
        uint4 wv[NS][2], sv[NS][2];
        const uint16_t* wrow = wr + (int64_t)e * H + (lane >> 4) * 16;
        const uint16_t* srow = scale + (lane >> 4) * 16;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int k = min(kt0 + s, nk - 1) * 64;
            wv[s][0] = reinterpret_cast<const uint4*>(wrow + k)[0];
            wv[s][1] = reinterpret_cast<const uint4*>(wrow + k)[1];
            sv[s][0] = reinterpret_cast<const uint4*>(srow + k)[0];
            sv[s][1] = reinterpret_cast<const uint4*>(srow + k)[1];
        }
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t w4[4] = {wv[s][h].x, wv[s][h].y, wv[s][h].z, wv[s][h].w};
                const uint32_t s4[4] = {sv[s][h].x, sv[s][h].y, sv[s][h].z, sv[s][h].w};
                uint32_t h4[4], l4[4];
                split_products8(w4, s4, h4, l4);
                bh[s][h] = make_uint4(h4[0], h4[1], h4[2], h4[3]);
                bl[s][h] = make_uint4(l4[0], l4[1], l4[2], l4[3]);
            }
    }
    for (int pass = 0; pass < T; pass += 16) {
        uint4 xa[NS][2];
        a_frags<NS>(x, H, min(pass + (lane & 15), T - 1), kt0, nk, lane, xa);
        f32x4_t c = {0.f, 0.f, 0.f, 0.f};
        float sq = 0.f;
#pragma unroll
        for (int s = 0; s < NS; ++s)
            if (s < n_steps) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    c = mfma16(xa[s][h], bh[s][h], c);
                    c = mfma16(xa[s][h], bl[s][h], c);
                    float f[8];
                    unpack8(xa[s][h], f);
#pragma unroll
                    for (int i = 0; i < 8; ++i) sq += f[i] * f[i];
                }
            }
        sq = tile_row_sum(sq);
        if (pass > 0) __syncthreads();  // the previous pass is done with red
        red_store(red, wave, 0, lane, c);
        if (lane < 16) red[kWaves * 512 + wave * 16 + lane] = sq;
        __syncthreads();
        const int r = tid >> 4, cc = tid & 15, t = pass + r, ee = nt * 16 + cc;
        if (t < T && ee < E) lpart[((int64_t)ks * T + t) * E + ee] = red_sum(red, 0, tid);
        if (nt == 0 && tid < 16 && pass + tid < T) {
            float v = red[kWaves * 512 + tid];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) v += red[kWaves * 512 + w * 16 + tid];
            ss_part[ks * T + pass + tid] = v;
        }
    }
}

// Router items first (ceil(E / 16) x kFrontSplit), then the dense gate/up
// items (Id / 16 x kFrontSplit) if with_dense and front_dense (else the
// routing launch runs them).
// Token items (one workgroup per token, first in the grid: the longest of the
// launch, so they start first) do what the token's row needs before the
// experts read it. The whole workgroup takes the row: lane l of wavefront w
// holds 8-value chunks l + 64 (w + 4 j) (hidden <= 4096), and its reductions
// go through DPP and then LDS in wavefront order.
//  - The layer's pre-norms (INF2 card, "The architecture (a dual-path FFN)"):
//    x_d = bf16(N_gd(h)) and x_m = bf16(N_gm(h)), N_g(v) = v / sqrt(mean(v^2)
//    + eps) * g, each where its gain is given. The router reads h itself, so
//    its items in this launch do not wait for them.
//  - E4M3 experts: the experts' input row (x_m, or x) quantised per row (max
//    |x| / 448, codes round half to even) into a.xq as half carriers, its
//    scale into a.x_scale[t].
__device__ __forceinline__ void front_token(const StreamArgs& a, int t, float* red) {
    constexpr int NC = 2;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nc = a.H >> 3;
    const uint16_t* row = a.pre_src ? a.pre_src : a.x;
    const uint4* src = reinterpret_cast<const uint4*>(row + (int64_t)t * a.H);
    uint4 v[NC];
    int cj[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        cj[j] = lane + kWave * (wave + kWaves * j);
        v[j] = src[min(cj[j], nc - 1)];  // clamped: a repeat of the last chunk
    }
    float f[NC][8];
#pragma unroll
    for (int j = 0; j < NC; ++j) unpack8(v[j], f[j]);
    if (a.pre_src) {
        uint4 gd[NC], gm[NC];
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            const int c = min(cj[j], nc - 1);
            gd[j] = a.pre_gd ? reinterpret_cast<const uint4*>(a.pre_gd)[c] : make_uint4(0u, 0u, 0u, 0u);
            gm[j] = a.pre_gm ? reinterpret_cast<const uint4*>(a.pre_gm)[c] : make_uint4(0u, 0u, 0u, 0u);
        }
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < NC; ++j)
            if (cj[j] < nc) {
#pragma unroll
                for (int i = 0; i < 8; ++i) ss += f[j][i] * f[j][i];
            }
        ss = wave_sum<kWave>(ss);
        if (lane == 0) red[wave] = ss;
        __syncthreads();
        float tot = red[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) tot += red[w];
        const float rn = 1.0f / sqrtf(tot / (float)a.H + a.pre_eps);
        __syncthreads();  // red is reused below
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            float g[8], o[8];
            if (a.pre_gd) {
                unpack8(gd[j], g);
#pragma unroll
                for (int i = 0; i < 8; ++i) o[i] = f[j][i] * rn * g[i];
                if (cj[j] < nc)
                    reinterpret_cast<uint4*>(a.pre_xd + (int64_t)t * a.H)[cj[j]] =
                        make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                                   pack_bf16x2(o[6], o[7]));
            }
            if (a.pre_gm) {
                unpack8(gm[j], g);
#pragma unroll
                for (int i = 0; i < 8; ++i) o[i] = f[j][i] * rn * g[i];
                const uint4 xm = make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                                            pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7]));
                if (cj[j] < nc) reinterpret_cast<uint4*>(a.pre_xm + (int64_t)t * a.H)[cj[j]] = xm;
                unpack8(xm, f[j]);  // the experts' input: x_m as rounded to bf16
            }
        }
    }
    if (!a.xq) return;
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < NC; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[j][i]));  // repeats: the same maximum
    amax = wave_max<kWave>(amax);
    if (lane == 0) red[wave] = amax;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) amax = fmaxf(amax, red[w]);
    const float s = amax / 448.0f;
    uint4* dst = reinterpret_cast<uint4*>(a.xq + (int64_t)t * a.H);
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        if (cj[j] < nc) {
            uint32_t o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t c0 = fp8_e4m3_code_div(f[j][2 * i], s);
                const uint32_t c1 = fp8_e4m3_code_div(f[j][2 * i + 1], s);
                o[i] = fp8_as_f16_bits(c0) | (fp8_as_f16_bits(c1) << 16);
            }
            dst[cj[j]] = make_uint4(o[0], o[1], o[2], o[3]);
        }
    }
    if (threadIdx.x == 0) a.x_scale[t] = s;
}

template <int NS>
__global__ __launch_bounds__(kThreads) void decode_front_kernel(StreamArgs a, const uint16_t* scale,
                                                               const uint16_t* wr, float* lpart,
                                                               float* ss_part) {
    __shared__ float red[kWaves * 512 + kWaves * 16];
    const int n_router = wr ? ((a.E + 15) / 16) * kFrontSplit : 0;
    const int n_dense = a.with_dense && a.front_dense ? (a.Id / 16) * kFrontSplit : 0;
    const int n_tok = (a.xq || a.pre_src) ? a.T : 0;  // token items first
    const int b = (int)blockIdx.x - n_tok;
    if (b < 0) {
        front_token(a, (int)blockIdx.x, red);
    } else if (b < n_router) {
        const int nt = b / kFrontSplit, ks = b - nt * kFrontSplit;
        router_part<NS>(a.xr, a.H, scale, wr, a.E, nt, ks, a.T, lpart, ss_part, red);
    } else if (b < n_router + n_dense) {
        const int i = b - n_router, hc = i / kFrontSplit, ks = i - hc * kFrontSplit;
        dense_gateup_part<NS>(a.xd, a.H, a.dgu, a.Id, hc, ks, a.T, a.dgu_part, red, (int)threadIdx.x);
    }
}

// Dense gate/up finish: hd[t][c] = gelu_tanh(gate) * up, each the sum of its
// kFrontSplit partial sums in split order; one thread per (t, c).
__device__ __forceinline__ void dense_finish(const StreamArgs& a, int blk) {
    const int i = blk * kThreads + threadIdx.x;
    if (i >= a.T * a.Id) return;
    const int t = i / a.Id, c = i - t * a.Id;
    float gp[kFrontSplit], up[kFrontSplit];
#pragma unroll
    for (int ks = 0; ks < kFrontSplit; ++ks) {
        const float* row = a.dgu_part + ((int64_t)ks * a.T + t) * 2 * a.Id;
        gp[ks] = row[c];
        up[ks] = row[a.Id + c];
    }
    float g = gp[0], u = up[0];
#pragma unroll
    for (int ks = 1; ks < kFrontSplit; ++ks) {
        g += gp[ks];
        u += up[ks];
    }
    a.hd[(int64_t)t * a.Id + c] = f32_to_bf16(gelu_tanh(g) * u);
}

// ---------------------------------------------------------------- K3
// Items of (touched expert, 16 h columns, half of the K range): twice as many
// workgroups of half the bytes, so that the last ones in flight finish sooner.
// Writes fp32 partial sums (hpart); the down kernel forms h from them.
template <int NS, int WQ>
__global__ __launch_bounds__(kThreads) void decode_experts_gateup_kernel(StreamArgs a) {
    extern __shared__ uint4 xs[];
    __shared__ float red[kWaves * kPass * 2 * 16];
    const int n_fin = a.with_dense ? (a.T * a.Id + kThreads - 1) / kThreads : 0;
    if ((int)blockIdx.x < n_fin) {
        dense_finish(a, (int)blockIdx.x);
        return;
    }
    const int b = (int)blockIdx.x - n_fin;
    const int ipe = a.I / 16;  // 16-column items per expert
    const int slot = b / (2 * ipe), rem = b - slot * 2 * ipe;
    const int hc = rem >> 1, half = rem & 1;
    if (slot >= *a.n_active) return;
    const int e = a.active[slot];
    const int p0 = a.offsets[e], n = a.offsets[e + 1] - p0;
    if (n <= 0) return;  // (an active expert has rows)
    const int64_t wstride = (int64_t)2 * a.I * a.H;
    const void* W = WQ ? (const void*)((const int8_t*)a.gu + e * wstride)
                         : (const void*)((const uint16_t*)a.gu + e * wstride);
    // E4M3 experts read x quantised per token (half carriers of value * 2^-8)
    gateup_half_item<NS, WQ>(WQ == 2 ? a.xq : a.x, (int64_t)a.T * a.H * 2, a.H, W, a.I, hc, half, a.perm_token + p0, n,
                               (int64_t)a.T * a.K * 2 * a.I, a.hpart + (int64_t)p0 * 2 * a.I, xs, red);
}

// ---------------------------------------------------------------- K2

// Workgroup 0 routes every token (ONNX export card, "Truthful graph
// contracts", row "Router"), the other workgroups finish the dense gate/up.
//
// Selection: one wavefront a token, the top K of its E logits by the
// wavefront top-k (descending logit, ties to the lower index), with the
// renormalised weights exp(l_k - l_0) / sum_j exp(l_j - l_0) over the K
// selected (the softmax denominator over all experts cancels), summed in k
// order, times the per-expert scale.
//
// Then the stable grouping by expert. With T <= 64 every token is one bit of a
// 64-bit mask per expert: the rank of pair (t, k) within its expert is the
// number of lower tokens in that expert's mask, the expert's row count its
// popcount.
// Top K of token t, run by one wavefront: the logits (the kFrontSplit slices of
// the router product and of the sum of squares added in slice order), then the
// wavefront top-k; lane k < K returns pair (t, k). Every load is issued before
// any is used (indices clamped to E - 1, lanes past E masked afterwards).
template <int NJ>
__device__ __forceinline__ void route_token(const float* __restrict__ lpart, const float* __restrict__ ss_part,
                                            const float* __restrict__ bias, const float* __restrict__ pes,
                                            int T, int E, int K, int H, float eps, float inv_sqrt_h, int t,
                                            int lane, int& ei, float& wt) {
    float sqv[kFrontSplit], lp[NJ][kFrontSplit], bv[NJ], pvl[NJ];
#pragma unroll
    for (int ks = 0; ks < kFrontSplit; ++ks) sqv[ks] = ss_part[ks * T + t];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int e = min(lane + kWave * j, E - 1);
#pragma unroll
        for (int ks = 0; ks < kFrontSplit; ++ks) lp[j][ks] = lpart[((int64_t)ks * T + t) * E + e];
        bv[j] = bias ? bias[e] : 0.f;
        pvl[j] = pes[e];
    }
    float sq = sqv[0];
#pragma unroll
    for (int ks = 1; ks < kFrontSplit; ++ks) sq += sqv[ks];
    // logit = (sum_h x s W) * rms(x)^-1 * H^-0.5 + bias
    const float f = (1.0f / sqrtf(sq / (float)H + eps)) * inv_sqrt_h;
    float lv[4] = {0.f, 0.f, 0.f, 0.f}, pv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        float acc = lp[j][0];
#pragma unroll
        for (int ks = 1; ks < kFrontSplit; ++ks) acc += lp[j][ks];
        lv[j] = acc * f + bv[j];
        pv[j] = pvl[j];
    }
    int ik[kMaxTopK];
    float wk[kMaxTopK];
    wave_topk_vals<true, NJ>(lv, pes, E, K, lane, ik, wk, pv);
    ei = ik[0];
    wt = wk[0];
#pragma unroll
    for (int k = 1; k < kMaxTopK; ++k)
        if (lane == k) {
            ei = ik[k];
            wt = wk[k];
        }
}

template <int NS>
__global__ __launch_bounds__(kRouteThreads) void decode_route_kernel(StreamArgs a, const float* lpart,
                                                                    const float* ss_part, const float* bias,
                                                                    const float* pes, float eps,
                                                                    float inv_sqrt_h, int32_t* topk_idx,
                                                                    float* topk_w) {
    if (!lpart || blockIdx.x > 0) {
        // dense gate/up items (they only need x), four 256-thread groups a workgroup
        __shared__ float red_d[4][kWaves * 512];
        const int grp = threadIdx.x >> 8;
        const int i = ((int)blockIdx.x - (lpart ? 1 : 0)) * 4 + grp;
        const int hc = i / kFrontSplit, ks = i - hc * kFrontSplit;
        dense_gateup_part<NS>(a.xd, a.H, a.dgu, a.Id, hc, ks, a.T, a.dgu_part, red_d[grp],
                              (int)threadIdx.x & 255);
        return;
    }
    __shared__ int s_idx[kMaxPairs];
    __shared__ float s_w[kMaxPairs];
    __shared__ unsigned long long s_mask[kMaxExperts];
    __shared__ int s_off[kMaxExperts + 1];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int T = a.T, K = a.K, E = a.E, TK = T * K;
    if (tid < E) s_mask[tid] = 0ull;
    // one wavefront a token
    for (int t = wave; t < T; t += kRouteThreads / kWave) {
        int ei;
        float wt;
        if (E <= 2 * kWave)
            route_token<2>(lpart, ss_part, bias, pes, T, E, K, a.H, eps, inv_sqrt_h, t, lane, ei, wt);
        else
            route_token<4>(lpart, ss_part, bias, pes, T, E, K, a.H, eps, inv_sqrt_h, t, lane, ei, wt);
        if (lane < K) {
            s_idx[t * K + lane] = ei;
            s_w[t * K + lane] = wt;
        }
    }
    // LDS-only barriers: no global store is waited on before the end
    lds_barrier();
    if (tid < TK) atomicOr(&s_mask[s_idx[tid]], 1ull << (tid / K));
    lds_barrier();
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
        // one scan of both: rows (<= 512) in the low half, active experts
        // (<= 256) in the high half
        const uint32_t sc = wave_incl_scan_u32((uint32_t)csum | ((uint32_t)asum << 16));
        const int ci = (int)(sc & 0xffffu), ai = (int)(sc >> 16);
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
    lds_barrier();
    if (tid < TK) {
        const int e = s_idx[tid], t = tid / K;
        const float wt = s_w[tid];
        const int pos = s_off[e] + __popcll(s_mask[e] & ((1ull << t) - 1ull));
        topk_idx[tid] = e;
        topk_w[tid] = wt;
        a.perm_token[pos] = t;
        a.perm_w[pos] = wt;
        a.inv_row[tid] = pos;
    }
}

// Rows p0 .. p0 + n / (I / 8) of h into LDS as [n_rows][I / 8] 16-byte chunks:
// h = gelu_tanh(gate) * up, gate and up each the sum of the two halves' fp32
// partial sums (times the int8 column scales), rounded to bf16. Loads are
// unconditional (indices clamped into range); only the LDS stores are predicated.
template <int KPER, int WQ>
__device__ __forceinline__ void stage_h(const StreamArgs& a, int p0, int n, const float* gs, uint4* hs) {
    const int I = a.I, hc8 = I >> 3;
    const int64_t half = (int64_t)a.T * a.K * 2 * I;
#pragma unroll
    for (int q = 0; q < KPER; ++q) {
        const int i = min((int)threadIdx.x + q * kThreads, n - 1);
        const int r = i / hc8, c = (i - r * hc8) * 8;
        const float* g0 = a.hpart + (int64_t)(p0 + r) * 2 * I + c;
        float gv[8], uv[8];
        {
            const float4 a0 = reinterpret_cast<const float4*>(g0)[0], a1 = reinterpret_cast<const float4*>(g0)[1];
            const float4 b0 = reinterpret_cast<const float4*>(g0 + half)[0], b1 = reinterpret_cast<const float4*>(g0 + half)[1];
            const float4 c0 = reinterpret_cast<const float4*>(g0 + I)[0], c1 = reinterpret_cast<const float4*>(g0 + I)[1];
            const float4 d0 = reinterpret_cast<const float4*>(g0 + half + I)[0], d1 = reinterpret_cast<const float4*>(g0 + half + I)[1];
            gv[0] = a0.x + b0.x; gv[1] = a0.y + b0.y; gv[2] = a0.z + b0.z; gv[3] = a0.w + b0.w;
            gv[4] = a1.x + b1.x; gv[5] = a1.y + b1.y; gv[6] = a1.z + b1.z; gv[7] = a1.w + b1.w;
            uv[0] = c0.x + d0.x; uv[1] = c0.y + d0.y; uv[2] = c0.z + d0.z; uv[3] = c0.w + d0.w;
            uv[4] = c1.x + d1.x; uv[5] = c1.y + d1.y; uv[6] = c1.z + d1.z; uv[7] = c1.w + d1.w;
        }
        uint32_t hw[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float g_lo = gv[2 * j], g_hi = gv[2 * j + 1], u_lo = uv[2 * j], u_hi = uv[2 * j + 1];
            if (WQ) {
                g_lo *= gs[c + 2 * j];
                g_hi *= gs[c + 2 * j + 1];
                u_lo *= gs[I + c + 2 * j];
                u_hi *= gs[I + c + 2 * j + 1];
            }
            hw[j] = pack_bf16x2(gelu_tanh(g_lo) * u_lo, gelu_tanh(g_hi) * u_hi);
        }
        const int ii = (int)threadIdx.x + q * kThreads;
        if (ii < n) hs[ii] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    }
}

// stage_h for int8 experts, four columns a thread and one 256-chunk round at
// a time: the down item keeps its widened weights in registers meanwhile, and
// this keeps the kernel within 128 registers (four wavefronts a SIMD).
// n4: chunks of 4 columns (rows p0 .. p0 + n4 / (I / 4)); same arithmetic as
// stage_h.
__device__ __forceinline__ void stage_h4_int8(const StreamArgs& a, int p0, int n4, const float* gs, uint4* hs) {
    const int I = a.I, hc4 = I >> 2;
    const int64_t half = (int64_t)a.T * a.K * 2 * I;
    uint2* hs2 = reinterpret_cast<uint2*>(hs);
#pragma unroll 1
    for (int i0 = 0; i0 < n4; i0 += kThreads) {
        const int i = min(i0 + (int)threadIdx.x, n4 - 1);
        const int r = i / hc4, c = (i - r * hc4) * 4;
        const float* g0 = a.hpart + (int64_t)(p0 + r) * 2 * I + c;
        const float4 ga = *reinterpret_cast<const float4*>(g0), gb = *reinterpret_cast<const float4*>(g0 + half);
        const float4 ua = *reinterpret_cast<const float4*>(g0 + I);
        const float4 ub = *reinterpret_cast<const float4*>(g0 + half + I);
        const float4 sg = *reinterpret_cast<const float4*>(gs + c), su = *reinterpret_cast<const float4*>(gs + I + c);
        const float g[4] = {(ga.x + gb.x) * sg.x, (ga.y + gb.y) * sg.y, (ga.z + gb.z) * sg.z, (ga.w + gb.w) * sg.w};
        const float u[4] = {(ua.x + ub.x) * su.x, (ua.y + ub.y) * su.y, (ua.z + ub.z) * su.z, (ua.w + ub.w) * su.w};
        if (i0 + (int)threadIdx.x < n4)
            hs2[i] = make_uint2(pack_bf16x2(gelu_tanh(g[0]) * u[0], gelu_tanh(g[1]) * u[1]),
                                pack_bf16x2(gelu_tanh(g[2]) * u[2], gelu_tanh(g[3]) * u[3]));
    }
}

// ---------------------------------------------------------------- K3b
// E4M3 experts: h of each routed pair (grouped row p) from the two K halves'
// partial sums, times the gate/up column scales and the token's activation
// scale (times 2^16: the two operands' half carriers hold value * 2^-8),
// h = gelu_tanh(gate) * up rounded to bf16, then quantised per row (max |h| /
// 448, codes round half to even: the recipe page's per-token activation
// quantisation) into a.h as half carriers, the row scale times 2^16 into
// a.h_scale. Workgroup b takes the rows of active expert b, a wavefront a row;
// a lane holds NC 8-column chunks.
template <int NC>
__global__ __launch_bounds__(kThreads) void decode_hquant_kernel(StreamArgs a) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if ((int)blockIdx.x >= *a.n_active) return;
    const int e = a.active[blockIdx.x];
    const int p0 = a.offsets[e], p1 = a.offsets[e + 1];
    const int I = a.I, hc8 = I >> 3;
    const int64_t half = (int64_t)a.T * a.K * 2 * I;
    const float* gs = a.gu_scale + (int64_t)e * 2 * I;
    for (int p = p0 + wave; p < p1; p += kWaves) {  // uniform per wavefront
        const float rs = a.x_scale[a.perm_token[p]] * 65536.f;
        const float* g0 = a.hpart + (int64_t)p * 2 * I;
        float hv[NC][8];
        float amax = 0.f;
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            const int c = min(lane + j * kWave, hc8 - 1) * 8;  // clamped: repeats a chunk, same max
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float g = (g0[c + i] + g0[half + c + i]) * gs[c + i] * rs;
                const float u = (g0[I + c + i] + g0[half + I + c + i]) * gs[I + c + i] * rs;
                hv[j][i] = bf16_to_f32(f32_to_bf16(gelu_tanh(g) * u));  // h rounded to bf16
                amax = fmaxf(amax, fabsf(hv[j][i]));
            }
        }
        amax = wave_max<kWave>(amax);
        const float s = amax / 448.0f;
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            const int cc = lane + j * kWave;
            if (cc < hc8) {
                uint32_t o[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t c0 = fp8_e4m3_code_div(hv[j][2 * i], s);
                    const uint32_t c1 = fp8_e4m3_code_div(hv[j][2 * i + 1], s);
                    o[i] = fp8_as_f16_bits(c0) | (fp8_as_f16_bits(c1) << 16);
                }
                reinterpret_cast<uint4*>(a.h + (int64_t)p * I)[cc] = make_uint4(o[0], o[1], o[2], o[3]);
            }
        }
        if (lane == 0) a.h_scale[p] = s * 65536.f;
    }
}

// ---------------------------------------------------------------- K4
// Down projections. A wavefront reads K-steps [kt0, kt0 + n_steps) (n_steps <=
// NS) of one 16-row tile of a tiled [H, inter] matrix and dots them with the
// token rows of h (or hd) staged in LDS; returns, in lanes 0..15, the partial
// sum of row lane of the tile for token n of the pass.
// (bf16 pieces, or 1-byte ones widened beforehand by widen_steps)
template <int NS, int WQ>
__device__ __forceinline__ float down_dot(const uint4 (&w)[NS][2], const uint16_t* hrow, int kt0, int n_steps,
                                          int lane) {
    const uint16_t* hp = hrow + kt0 * 64 + (lane >> 4) * 16;
    float acc = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s)
        if (s < n_steps) acc = wide_dot<WQ>(w[s], hp + s * 64, acc);
    return tile_row_sum(acc);
}

// DMA loads a wavefront issues per pass: the E4M3 h rows of a pass, the dense
// rows of a pass (I <= 64 NS, Id <= 256 NS). (bf16 and int8 experts form h
// from the two K halves' partial sums as they stage it: their loads, issued
// right behind the weights, land right behind them without a copy to LDS
// first.)
template <int NS>
constexpr int kDownRowQ = (kPass * 8 * NS + kThreads - 1) / kThreads;
template <int NS>
constexpr int kDenseRowQ = (kPass * 32 * NS + kThreads - 1) / kThreads;

template <int NS, int WQ>
__global__ __launch_bounds__(kThreads) void decode_down_kernel(StreamArgs a) {
    extern __shared__ uint4 hs[];  // [kPass][max(I, Id)] bf16 (rounded up to whole DMA loads)
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
        if (n_rows <= 0) return;  // (an active expert has rows)
        const int64_t wstride = (int64_t)a.H * a.I;
        const char* W = WQ ? (const char*)((const int8_t*)a.dw + e * wstride)
                             : (const char*)((const uint16_t*)a.dw + e * wstride);
        const int nk = a.I >> 6, tile = g * kWaves + wave;
        const int hc8 = a.I >> 3;
        // E4M3: the pass's rows' activation scales (the first pass's read
        // ahead of everything, on the scalar path), and its rows of h -> LDS,
        // issued right behind the weights
        QuadOf<float> hsc{1.f, 1.f, 1.f, 1.f};
        if constexpr (WQ == 2) hsc = QuadOf<float>::load(a.h_scale + p0, min(kPass, n_rows));
        const int pairs = a.T * a.K;  // grouped rows
        auto stage = [&](int pass, int nt) {
            const int o0 = (p0 + pass) * a.I * 2;
            dma_chunks<kDownRowQ<NS>>(hs, nt * hc8, a.h, (int64_t)pairs * a.I * 2, [&](int j) { return o0 + j * 16; });
        };
        uint4 w[NS][WQ ? 1 : 2];
        tile_load<NS, WQ>(W + (int64_t)tile * nk * kTileBytes<WQ>, 0, nk, lane, w);
        if constexpr (WQ == 2) stage(0, min(kPass, n_rows));
        uint4 ww[NS][2];  // 1-byte weights: widened as they land
        if constexpr (WQ != 0) widen_steps<NS, WQ>(w, ww);
        const float sc = WQ ? a.dw_scale[(int64_t)e * a.H + tile * 16 + (lane & 15)] : 1.f;
        const float* gs = WQ ? a.gu_scale + (int64_t)e * 2 * a.I : nullptr;
        for (int pass = 0; pass < n_rows; pass += kPass) {
            const int nt = min(kPass, n_rows - pass);
            if constexpr (WQ == 2) {
                if (pass > 0) {
                    __syncthreads();  // previous pass done with hs
                    stage(pass, nt);
                    hsc = QuadOf<float>::load(a.h_scale + p0 + pass, nt);
                }
                dma_wait();
                __syncthreads();
            } else {
                __syncthreads();
                if constexpr (WQ == 1) stage_h4_int8(a, p0 + pass, nt * (a.I >> 2), gs, hs);
                else stage_h<(kPass * 128 + kThreads - 1) / kThreads, WQ>(a, p0 + pass, nt * hc8, gs, hs);
                __syncthreads();
            }
#pragma unroll 1
            for (int n = 0; n < nt; ++n) {
                const uint16_t* hrow = reinterpret_cast<const uint16_t*>(hs + n * hc8);
                float v;
                if constexpr (WQ != 0) v = down_dot<NS, WQ>(ww, hrow, 0, nk, lane);
                else v = down_dot<NS, 0>(w, hrow, 0, nk, lane);
                const float hv = WQ == 2 ? hsc.pick(n) : 1.f;
                if (lane < 16) a.part[(int64_t)(p0 + pass + n) * a.H + tile * 16 + lane] = v * sc * hv;
            }
        }
    } else {
        // dense down: one 16-row tile per workgroup, K split over the wavefronts
        const int tile = (int)blockIdx.x;
        const int nk = a.Id >> 6, kd = (nk + kWaves - 1) / kWaves;
        const int kt0 = wave * kd, n_steps = max(0, min(kd, nk - kt0));
        const int hc8 = a.Id >> 3;
        auto stage = [&](int pass, int nt) {
            const int o0 = pass * a.Id * 2;
            dma_chunks<kDenseRowQ<NS>>(hs, nt * hc8, a.hd, (int64_t)a.T * a.Id * 2, [&](int j) { return o0 + j * 16; });
        };
        uint4 w[NS][2];
        tile_load<NS, false>(reinterpret_cast<const char*>(a.ddw) + (int64_t)tile * nk * kTileBytes<false>,
                             kt0, nk, lane, w);
        stage(0, min(kPass, a.T));
        for (int pass = 0; pass < a.T; pass += kPass) {
            const int nt = min(kPass, a.T - pass);
            if (pass > 0) {
                __syncthreads();  // previous pass done with hs and red
                stage(pass, nt);
            }
            dma_wait();
            __syncthreads();
#pragma unroll 1
            for (int n = 0; n < nt; ++n) {
                const float v = down_dot<NS, 0>(w, reinterpret_cast<const uint16_t*>(hs + n * hc8),
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
        // the router weight of pair (t, k) (the same value as perm_w of its
        // grouped row), loaded beside the inverse rows rather than after them
        float wk[kMaxTopK];
#pragma unroll
        for (int k = 0; k < kMaxTopK; ++k) wk[k] = a.topk_w[(int64_t)t * a.K + min(k, a.K - 1)];
        float4 r[kMaxTopK];
#pragma unroll
        for (int k = 0; k < kMaxTopK; ++k) r[k] = *reinterpret_cast<const float4*>(a.part + (int64_t)p[k] * a.H + c);
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

template <int NS>
hipError_t launch_front_ns(const StreamArgs& a, const uint16_t* scale, const uint16_t* wr, float* lpart,
                           float* ss_part, hipStream_t stream) {
    const int n_router = wr ? ((a.E + 15) / 16) * kFrontSplit : 0;
    const int n_tok = (a.xq || a.pre_src) ? a.T : 0;  // token items: pre-norms, E4M3 quantisation
    const int blocks = n_router + (a.with_dense && a.front_dense ? (a.Id / 16) * kFrontSplit : 0) + n_tok;
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(decode_front_kernel<NS>, dim3(blocks), dim3(kThreads), 0, stream, a, scale, wr, lpart,
                       ss_part);
    return hipGetLastError();
}

template <int NJ>
hipError_t launch_experts_nj(const StreamArgs& a, int wq, hipStream_t stream) {
    const int n_fin = a.with_dense ? (a.T * a.Id + kThreads - 1) / kThreads : 0;
    const int blocks = n_fin + a.max_active * (a.I / 16) * 2;
    if (blocks <= 0) return hipSuccess;
    // a pass's x rows (half the hidden size each), rounded up to whole DMA loads
    const size_t kq = (kPass * 32 * NJ + kThreads - 1) / kThreads;
    const size_t x_bytes = (size_t)kPass * (a.H / 2) * sizeof(uint16_t), dma_bytes = kq * kThreads * sizeof(uint4);
    const size_t lds = x_bytes > dma_bytes ? x_bytes : dma_bytes;
    if (wq == 2)
        hipLaunchKernelGGL((decode_experts_gateup_kernel<NJ, 2>), dim3(blocks), dim3(kThreads), lds, stream, a);
    else if (wq == 1)
        hipLaunchKernelGGL((decode_experts_gateup_kernel<NJ, 1>), dim3(blocks), dim3(kThreads), lds, stream, a);
    else
        hipLaunchKernelGGL((decode_experts_gateup_kernel<NJ, 0>), dim3(blocks), dim3(kThreads), lds, stream, a);
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

hipError_t launch_decode_front(const StreamArgs& a, const uint16_t* scale, const uint16_t* wr, float* lpart,
                               float* ss_part, hipStream_t stream) {
    // K-steps per wavefront: the H / 64 steps over kFrontSplit workgroups of four
    switch ((a.H / 64 + kFrontSplit * kWaves - 1) / (kFrontSplit * kWaves)) {
        case 1: return launch_front_ns<1>(a, scale, wr, lpart, ss_part, stream);
        case 2: return launch_front_ns<2>(a, scale, wr, lpart, ss_part, stream);
        case 3: return launch_front_ns<3>(a, scale, wr, lpart, ss_part, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int NS>
hipError_t launch_route_ns(const StreamArgs& a, const float* lpart, const float* ss_part, const float* bias,
                           const float* pes, float eps, int32_t* topk_idx, float* topk_w, hipStream_t stream) {
    // the dense items, four a workgroup ((Id / 16) * kFrontSplit is a multiple of 4)
    const int n_dense = (a.with_dense && !a.front_dense) ? (a.Id / 16) * kFrontSplit / 4 : 0;
    const int blocks = (lpart ? 1 : 0) + n_dense;
    if (blocks <= 0) return hipSuccess;
    const float inv_sqrt_h = (float)(1.0 / __builtin_sqrt((double)a.H));
    hipLaunchKernelGGL(decode_route_kernel<NS>, dim3(blocks), dim3(kRouteThreads), 0, stream, a, lpart, ss_part,
                       bias, pes, eps, inv_sqrt_h, topk_idx, topk_w);
    return hipGetLastError();
}

hipError_t launch_decode_route(const StreamArgs& a, const float* lpart, const float* ss_part, const float* bias,
                               const float* pes, float eps, int32_t* topk_idx, float* topk_w,
                               hipStream_t stream) {
    static_assert(kFrontSplit % 4 == 0, "dense items come four a workgroup");
    switch ((a.H / 64 + kFrontSplit * kWaves - 1) / (kFrontSplit * kWaves)) {
        case 1: return launch_route_ns<1>(a, lpart, ss_part, bias, pes, eps, topk_idx, topk_w, stream);
        case 2: return launch_route_ns<2>(a, lpart, ss_part, bias, pes, eps, topk_idx, topk_w, stream);
        case 3: return launch_route_ns<3>(a, lpart, ss_part, bias, pes, eps, topk_idx, topk_w, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_experts_gateup(const StreamArgs& a, int wq, hipStream_t stream) {
    // K-steps per wavefront: half of the H / 64 steps over four wavefronts
#define CALL(n) launch_experts_nj<n>(a, wq, stream)
    MOE_NJ_SWITCH((a.H / 128 + kWaves - 1) / kWaves, CALL)
#undef CALL
}

// LDS of a down workgroup: the larger of an expert item's (h rows; E4M3
// rounded up to whole DMA loads) and a dense item's (its rows, rounded up
// likewise)
template <int NS>
size_t down_lds_bytes(const StreamArgs& a, int wq) {
    const size_t rows = (size_t)kPass * (a.I / 8);
    size_t chunks = wq == 2 ? std::max(rows, (size_t)kDownRowQ<NS> * kThreads) : rows;
    if (a.with_dense) chunks = std::max(chunks, std::max((size_t)kPass * (a.Id / 8), (size_t)kDenseRowQ<NS> * kThreads));
    return chunks * sizeof(uint4);
}

hipError_t launch_decode_down(const StreamArgs& a, int wq, hipStream_t stream) {
    // K-steps a wavefront holds: a whole expert tile (I / 64) or a quarter of
    // a dense tile (Id / 256, rounded up)
    const int need = max(a.I / 64, (a.Id / 64 + kWaves - 1) / kWaves);
    const int blocks = a.max_active * (a.H / 64) + (a.with_dense ? a.H / 16 : 0);
    if (blocks <= 0) return hipSuccess;
    const dim3 grid(blocks), block(kThreads);
#define LAUNCH(N)                                                                                   \
    do {                                                                                            \
        const size_t lds = down_lds_bytes<N>(a, wq);                                                \
        if (wq == 2) hipLaunchKernelGGL((decode_down_kernel<N, 2>), grid, block, lds, stream, a);   \
        else if (wq == 1) hipLaunchKernelGGL((decode_down_kernel<N, 1>), grid, block, lds, stream, a); \
        else hipLaunchKernelGGL((decode_down_kernel<N, 0>), grid, block, lds, stream, a);            \
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

hipError_t launch_decode_hquant(const StreamArgs& a, hipStream_t stream) {
    const int blocks = a.max_active;
    if (blocks <= 0) return hipSuccess;
    const int nc = (a.I / 8 + kWave - 1) / kWave;  // 8-column chunks per lane
#define LAUNCH(N)                                                                                    \
    do {                                                                                             \
        hipLaunchKernelGGL(decode_hquant_kernel<N>, dim3(blocks), dim3(kThreads), 0, stream, a);     \
        return hipGetLastError();                                                                    \
    } while (0)
    if (nc <= 1) LAUNCH(1);
    if (nc <= 2) LAUNCH(2);
#undef LAUNCH
    return hipErrorInvalidValue;  // expert_inter <= 1024 on the streaming path
}

hipError_t launch_decode_combine(const StreamArgs& a, hipStream_t stream) {
    const int n = a.T * (a.H / 4);
    hipLaunchKernelGGL(decode_combine_kernel, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace moe
