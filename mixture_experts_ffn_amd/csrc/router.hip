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
// router_tile_kernel: a workgroup takes 16 NRT tokens and one slice of the
//   hidden dimension. Wavefront w owns the 16-expert column tiles w, w + 4, ...:
//   it loads its router rows straight from global memory in the MFMA operand
//   layout, forms s*W and splits it into hi and lo in registers, so each router
//   row is read once per workgroup and never staged. The x tile [16 NRT][64]
//   of each K-step moves from global memory straight into LDS
//   (global_load_lds_dwordx4) and is read by all four wavefronts; wavefront w
//   also accumulates the sums of squares of the row tiles r with r % 4 == w
//   from the fragments it reads. Both operands run three K-steps ahead (four
//   LDS stages of x, a four-slot register ring of router fragments), with one
//   exact wait and one barrier a step. Outputs: partial[slice][t][e] and
//   ss_partial[slice][t].
// router_finish_kernel: one wavefront per token adds the slices in order (the
//   same order for every run), applies the RMSNorm factor from the slices'
//   sums of squares (x is not read again), the H^-0.5 and the bias, and runs
//   the softmax / top-k.
namespace {

constexpr int kRK = 64;  // K-step
constexpr int kRThreads = 256;
constexpr int kRMinSliceSteps = 4;  // a slice's partial sums are written once per K range of at least this

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// LDS position of 16-byte chunk c of x tile row r: chunk c ^ f(r), f(r) =
// (r & 7) ^ ((r >> 3) & 1). 128-bit reads of chunk c of 16 consecutive rows
// (one cycle's 16 lanes over 64 banks) then hit 16 distinct (row parity,
// chunk) bank groups.
__device__ __forceinline__ int rsw(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int rswz(int r, int c) { return r * kRK + ((c ^ rsw(r)) << 3); }

__device__ __forceinline__ v4u ld16(const uint16_t* p) { return *reinterpret_cast<const v4u*>(p); }

// one K-step of a lane's router fragments: NCW column tiles x two 32-wide k
// blocks, and the matching 8 router-scale values of each block
template <int NCW>
struct RSlot {
    v4u w[NCW][2];
    v4u sc[2];
};

// s_waitcnt vmcnt(n) lgkmcnt(0) (vmcnt split over bits 3:0 and 15:14)
constexpr int r_wait_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

template <int NCW, int NRT>
__global__ __launch_bounds__(kRThreads) void router_tile_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ scale,
    const uint16_t* __restrict__ w, int T, int H, int E, int slice_steps,
    float* __restrict__ partial, float* __restrict__ ss_partial) {
    constexpr int kTok = 16 * NRT;             // tokens per workgroup
    constexpr int NXC = kTok * 8 / kRThreads;  // 1 KB direct loads of x a wavefront issues per K-step
    constexpr int kLoads = NXC + 2 * NCW + 2;  // loads a lane issues per K-step
    static_assert(2 * kLoads < 64, "vmcnt range");
    // four distinct stages (so that the compiler can tell which one a pending direct load writes)
    __shared__ __attribute__((aligned(16))) uint16_t xs0[kTok * kRK];
    __shared__ __attribute__((aligned(16))) uint16_t xs1[kTok * kRK];
    __shared__ __attribute__((aligned(16))) uint16_t xs2[kTok * kRK];
    __shared__ __attribute__((aligned(16))) uint16_t xs3[kTok * kRK];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int t0 = blockIdx.x * kTok;
    const int nt = min(kTok, T - t0);
    const int n_ct = (E + 15) / 16;
    const int nk = H / kRK;
    const int kb = blockIdx.y * slice_steps, n = min(nk, kb + slice_steps) - kb;

    // x: direct load q of wavefront w covers tile rows 8 (w NXC + q) .. + 8,
    // lane l landing in row l / 8 at physical chunk l % 8, so it fetches
    // logical chunk (l % 8) ^ f(row) (rows past the batch repeat its last row)
    const uint16_t* xp[NXC];
#pragma unroll
    for (int q = 0; q < NXC; ++q) {
        const int r = (wave * NXC + q) * 8 + (lane >> 3);
        xp[q] = x + (int64_t)(t0 + min(r, nt - 1)) * H + (int64_t)kb * kRK + (((lane & 7) ^ rsw(r)) << 3);
    }
    // router fragments: row ct * 16 + lane % 16 of column tile ct = wave + 4 c,
    // k = 8 (lane / 16) .. + 8 of each 32-wide block (rows past E repeat row E - 1)
    const uint16_t* wp[NCW];
#pragma unroll
    for (int c = 0; c < NCW; ++c)
        wp[c] = w + (int64_t)min((wave + 4 * c) * 16 + (lane & 15), E - 1) * H + (int64_t)kb * kRK + (lane >> 4) * 8;
    const uint16_t* sp = scale + (int64_t)kb * kRK + (lane >> 4) * 8;

    auto issue = [&](int j, uint16_t* st, RSlot<NCW>& rs) {
        const int64_t off = (int64_t)j * kRK;
        asm volatile("" ::: "memory");
#pragma unroll
        for (int q = 0; q < NXC; ++q)
            __builtin_amdgcn_global_load_lds((glb_void_t*)(xp[q] + off),
                                             (lds_void_t*)(st + (wave * NXC + q) * 8 * kRK), 16, 0, 0);
#pragma unroll
        for (int c = 0; c < NCW; ++c) {
            rs.w[c][0] = ld16(wp[c] + off);
            rs.w[c][1] = ld16(wp[c] + off + 32);
        }
        rs.sc[0] = ld16(sp + off);
        rs.sc[1] = ld16(sp + off + 32);
        asm volatile("" ::: "memory");
    };

    f32x4_t acc[NRT][NCW];
#pragma unroll
    for (int r = 0; r < NRT; ++r)
#pragma unroll
        for (int c = 0; c < NCW; ++c) acc[r][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float ss[(NRT + 3) / 4];  // row tiles wave, wave + 4, ...: this lane's share of row lane % 16
#pragma unroll
    for (int i = 0; i < (NRT + 3) / 4; ++i) ss[i] = 0.f;

    auto compute = [&](const uint16_t* st, const RSlot<NCW>& rs) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            bf16x8_t bh[NCW], bl[NCW];
#pragma unroll
            for (int c = 0; c < NCW; ++c) {
                const uint32_t wa[4] = {rs.w[c][s][0], rs.w[c][s][1], rs.w[c][s][2], rs.w[c][s][3]};
                const uint32_t sa[4] = {rs.sc[s][0], rs.sc[s][1], rs.sc[s][2], rs.sc[s][3]};
                uint32_t h[4], l[4];
                split_products8(wa, sa, h, l);
                bh[c] = __builtin_bit_cast(bf16x8_t, v4u{h[0], h[1], h[2], h[3]});
                bl[c] = __builtin_bit_cast(bf16x8_t, v4u{l[0], l[1], l[2], l[3]});
            }
            const int ch = s * 4 + (lane >> 4);
#pragma unroll
            for (int r = 0; r < NRT; ++r) {
                const v4u av = *reinterpret_cast<const v4u*>(st + rswz(r * 16 + (lane & 15), ch));
                if ((r & 3) == wave) {  // uniform
                    float f[8];
                    unpack8(make_uint4(av[0], av[1], av[2], av[3]), f);
#pragma unroll
                    for (int q = 0; q < 8; ++q) ss[r >> 2] += f[q] * f[q];
                }
                const bf16x8_t af = __builtin_bit_cast(bf16x8_t, av);
#pragma unroll
                for (int c = 0; c < NCW; ++c) {
                    if (wave + 4 * c < n_ct) {  // uniform
                        acc[r][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bh[c], acc[r][c], 0, 0, 0);
                        acc[r][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bl[c], acc[r][c], 0, 0, 0);
                    }
                }
            }
        }
    };

    RSlot<NCW> r0, r1, r2, r3;
    issue(0, xs0, r0);
    if (n > 1) issue(1, xs1, r1);
    if (n > 2) issue(2, xs2, r2);
    // step i: wait until only this lane's loads of the (at most two) later
    // steps already issued are pending (its share of step i has landed),
    // barrier (every lane's share has; every wavefront is done with step i-1,
    // whose stage and slot step i+3 reuses), issue step i+3 if the slice has
    // it, multiply step i.
#define MOE_ROUTER_STEP(U, SC, RC, SN, RN)                                                  \
    {                                                                                       \
        const int i = j + (U), ahead = n - 1 - i;                                           \
        if (ahead >= 2) __builtin_amdgcn_s_waitcnt(r_wait_vm(2 * kLoads));                  \
        else if (ahead == 1) __builtin_amdgcn_s_waitcnt(r_wait_vm(kLoads));                 \
        else __builtin_amdgcn_s_waitcnt(r_wait_vm(0));                                      \
        raw_barrier();                                                                      \
        if (i + 3 < n) issue(i + 3, SN, RN);                                                \
        if (i < n) compute(SC, RC);                                                         \
    }
    for (int j = 0; j < n; j += 4) {
        MOE_ROUTER_STEP(0, xs0, r0, xs3, r3)
        MOE_ROUTER_STEP(1, xs1, r1, xs0, r0)
        MOE_ROUTER_STEP(2, xs2, r2, xs1, r1)
        MOE_ROUTER_STEP(3, xs3, r3, xs2, r2)
    }
#undef MOE_ROUTER_STEP
    __builtin_amdgcn_s_waitcnt(7 << 4);  // vmcnt(0) lgkmcnt(0): no direct load still writing LDS

    // each row's sum of squares over the slice: the four lanes l % 16 + 16 i
    // hold its four k quarters, added in a fixed order
#pragma unroll
    for (int i = 0; i < (NRT + 3) / 4; ++i) {
        float v = ss[i];
        v += __shfl_xor(v, 16, kWave);
        v += __shfl_xor(v, 32, kWave);
        const int row = (wave + 4 * i) * 16 + lane;
        if (wave + 4 * i < NRT && lane < 16 && row < nt) ss_partial[(int64_t)blockIdx.y * T + t0 + row] = v;
    }

    float* out = partial + (int64_t)blockIdx.y * T * E;
#pragma unroll
    for (int c = 0; c < NCW; ++c) {
        const int ct = wave + 4 * c;
        const int e = ct * 16 + (lane & 15);
        if (ct < n_ct && e < E) {
#pragma unroll
            for (int r = 0; r < NRT; ++r)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int row = r * 16 + (lane >> 4) * 4 + v;
                    if (row < nt) out[(int64_t)(t0 + row) * E + e] = acc[r][c][v];
                }
        }
    }
}

// tokens per workgroup: 128 once there are enough of them to fill the chip
// with whole-K-range slices of a few K-steps, else 64 (more workgroups)
int router_tile_tokens(int T, int E) { return (E <= 128 && T >= 8192) ? 128 : 64; }

}  // namespace

// Slices are read eight at a time, all eight loads issued before the first is
// added (the sums stay in slice order); the per-expert scales are loaded
// beside them, so that nothing waits on the selection.
template <int NJ>
__global__ __launch_bounds__(256) void router_finish_kernel(
    const float* __restrict__ partial, const float* __restrict__ ss_partial, int S,
    const float* __restrict__ bias, const float* __restrict__ pes, int T, int H, int E, int K,
    float eps, float inv_sqrt_h, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
    constexpr int kBatch = 8;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;  // uniform per wavefront
    float lv[4] = {0.f, 0.f, 0.f, 0.f}, pv[4] = {0.f, 0.f, 0.f, 0.f}, bv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int e = min(lane + kWave * j, E - 1);
        pv[j] = pes[e];
        if (bias) bv[j] = bias[e];
    }
    float q = 0.f;  // sum of squares of x_t: the slices' shares, in slice order
    for (int s0 = 0; s0 < S; s0 += kBatch) {
        float v[kBatch][NJ], sq[kBatch];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const int64_t sl = min(s0 + b, S - 1);
#pragma unroll
            for (int j = 0; j < NJ; ++j) v[b][j] = partial[(sl * T + t) * E + min(lane + kWave * j, E - 1)];
            sq[b] = ss_partial[sl * T + t];
        }
#pragma unroll
        for (int b = 0; b < kBatch; ++b)
            if (s0 + b < S) {
#pragma unroll
                for (int j = 0; j < NJ; ++j) lv[j] += v[b][j];
                q += sq[b];
            }
    }
    const float f = (1.0f / sqrtf(q / (float)H + eps)) * inv_sqrt_h;
#pragma unroll
    for (int j = 0; j < NJ; ++j) lv[j] = lv[j] * f + bv[j];
    int ik[kMaxTopK];
    float wk[kMaxTopK];
    wave_topk_vals<true, NJ>(lv, pes, E, K, lane, ik, wk, pv);
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k)
        if (k < K && lane == k) {
            topk_idx[(int64_t)t * K + k] = ik[k];
            topk_w[(int64_t)t * K + k] = wk[k];
        }
}

RouterSplit router_split(int T, int H, int E) {
    const int tok = router_tile_tokens(T, E);
    const int n_tiles = (T + tok - 1) / tok;
    const int nk = H / kRK;
    // about two workgroups per CU; slices of at least kRMinSliceSteps K-steps
    int S = (512 + n_tiles - 1) / n_tiles;
    S = S < 1 ? 1 : S;
    const int max_s = (nk + kRMinSliceSteps - 1) / kRMinSliceSteps;
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
    const int tok = router_tile_tokens(T, E);
    const dim3 grid((T + tok - 1) / tok, rs.slices);
    // partial: the slices' logit sums [S][T][E], then their sums of squares [S][T]
    float* ss_partial = partial + (int64_t)rs.slices * T * E;
    if (E > 128)
        hipLaunchKernelGGL((router_tile_kernel<4, 4>), grid, dim3(kRThreads), 0, stream, x, scale, w, T, H, E,
                           rs.slice_steps, partial, ss_partial);
    else if (tok == 128)
        hipLaunchKernelGGL((router_tile_kernel<2, 8>), grid, dim3(kRThreads), 0, stream, x, scale, w, T, H, E,
                           rs.slice_steps, partial, ss_partial);
    else
        hipLaunchKernelGGL((router_tile_kernel<2, 4>), grid, dim3(kRThreads), 0, stream, x, scale, w, T, H, E,
                           rs.slice_steps, partial, ss_partial);
    const dim3 fgrid((T + 3) / 4);
#define MOE_FINISH(NJ)                                                                                   \
    hipLaunchKernelGGL(router_finish_kernel<NJ>, fgrid, dim3(256), 0, stream, partial, ss_partial, rs.slices, \
                       bias, pes, T, H, E, K, eps, inv_sqrt_h, topk_idx, topk_w)
    if (E <= 64) MOE_FINISH(1);
    else if (E <= 128) MOE_FINISH(2);
    else if (E <= 192) MOE_FINISH(3);
    else MOE_FINISH(4);
#undef MOE_FINISH
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
