// Expert grouping of the routed (token, slot) pairs on gfx950.
//
// Gathered expert compute (Tenstorrent bundle card, "Configurable knobs",
// GEMMA4_PREFILL_GATHERED) runs each expert only on the tokens routed to it.
// This kernel builds that grouping: a stable counting sort of the T*K pairs by
// expert (ascending expert, then ascending token), with
//   counts[e], offsets[e] (exclusive prefix sum), perm_token / perm_w (token and
//   router weight of each grouped row), inv_row[t*K+k] (grouped row of a pair),
//   the list of experts with rows, and the list of BM-row tiles for the
//   grouped GEMMs.
// It is exact integer work, and deterministic: ranks within an expert come from
// bit masks of the lanes of a 64-token tile that picked the expert (popcount of
// the lower lanes), never from the order of atomic operations.
//
// One workgroup of 1024 threads handles the whole batch; tokens are taken in
// tiles of 64 (one lane per token, one wavefront per tile).
#include "common.h"
#include "kernels.h"
#include "topk.h"

namespace moe {

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / kWave;

__global__ __launch_bounds__(kPermThreads) void permute_kernel(
    const float* __restrict__ logits, const float* __restrict__ pes, int32_t* topk_idx,
    float* topk_w, int T, int K, int E, int BM, PermuteOut o) {
    __shared__ unsigned long long mask[kPermWaves][kMaxExperts];  // 32 KB
    __shared__ int part[kPermThreads];
    __shared__ int s_cnt[kMaxExperts];
    __shared__ int s_off[kMaxExperts + 1];
    __shared__ int s_tile[kMaxExperts + 1];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

    // fused top-k for small batches
    if (logits) {
        for (int t = wave; t < T; t += kPermWaves) {
            int ik[kMaxTopK];
            float wk[kMaxTopK];
            wave_topk(logits + (size_t)t * E, pes, E, K, lane, ik, wk);
            if (lane == 0) {
#pragma unroll
                for (int k = 0; k < kMaxTopK; ++k)
                    if (k < K) {
                        topk_idx[(size_t)t * K + k] = ik[k];
                        topk_w[(size_t)t * K + k] = wk[k];
                    }
            }
        }
        block_sync_global();
    }

    const int n_tiles = (T + 63) / 64;
    // phase 1: experts picked by each 64-token tile, as lane masks -> counts
    for (int base = 0; base < n_tiles; base += kPermWaves) {
        const int tile = base + wave;
        for (int e = lane; e < E; e += kWave) mask[wave][e] = 0ull;
        __syncthreads();
        const int t = tile * 64 + lane;
        if (tile < n_tiles && t < T) {
            for (int k = 0; k < K; ++k)
                atomicOr(&mask[wave][topk_idx[(size_t)t * K + k]], 1ull << lane);
        }
        __syncthreads();
        if (tile < n_tiles)
            for (int e = lane; e < E; e += kWave)
                o.tile_counts[(size_t)tile * E + e] = __popcll(mask[wave][e]);
        __syncthreads();
    }
    block_sync_global();

    // phase 2: totals, offsets and the base row of every (tile, expert)
    int ep = 1;
    while (ep < E) ep <<= 1;
    const int nparts = kPermThreads / ep;
    const int e = tid & (ep - 1), p = tid / ep;
    const int chunk = (n_tiles + nparts - 1) / nparts;
    const int tb = min(n_tiles, p * chunk), te = min(n_tiles, tb + chunk);
    {
        int sum = 0;
        if (e < E) {
#pragma unroll 8
            for (int tl = tb; tl < te; ++tl) sum += o.tile_counts[(size_t)tl * E + e];
        }
        part[tid] = sum;
    }
    __syncthreads();
    if (wave == 0) {
        // lane l owns experts 4l .. 4l+3
        int c[4], nt_e[4], act[4];
        int csum = 0, tsum = 0, asum = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ee = lane * 4 + i;
            int cnt = 0;
            if (ee < E)
                for (int q = 0; q < nparts; ++q) cnt += part[q * ep + ee];
            c[i] = cnt;
            nt_e[i] = (cnt + BM - 1) / BM;
            act[i] = (cnt > 0) ? 1 : 0;
            csum += c[i];
            tsum += nt_e[i];
            asum += act[i];
        }
        int ci = csum, ti = tsum, ai = asum;  // inclusive scans across lanes
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int a = __shfl_up(ci, off, kWave), b = __shfl_up(ti, off, kWave),
                      d = __shfl_up(ai, off, kWave);
            if (lane >= off) {
                ci += a;
                ti += b;
                ai += d;
            }
        }
        int crun = ci - csum, trun = ti - tsum, arun = ai - asum;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ee = lane * 4 + i;
            if (ee < E) {
                s_cnt[ee] = c[i];
                s_off[ee] = crun;
                s_tile[ee] = trun;
                o.counts[ee] = c[i];
                o.offsets[ee] = crun;
                if (act[i]) o.active[arun] = ee;
            }
            crun += c[i];
            trun += nt_e[i];
            arun += act[i];
        }
        if (lane == kWave - 1) {
            s_off[E] = ci;
            s_tile[E] = ti;
            o.offsets[E] = ci;
            *o.n_mtiles = ti;
            *o.n_active = ai;
        }
    }
    __syncthreads();
    if (e < E) {
        int run = s_off[e];
        for (int q = 0; q < p; ++q) run += part[q * ep + e];
#pragma unroll 8
        for (int tl = tb; tl < te; ++tl) {
            const size_t ix = (size_t)tl * E + e;
            const int cnt = o.tile_counts[ix];
            o.tile_counts[ix] = run;
            run += cnt;
        }
    }
    // tiles of BM grouped rows for the grouped GEMMs
    for (int ee = tid; ee < E; ee += kPermThreads) {
        const int nt = (s_cnt[ee] + BM - 1) / BM;
        for (int j = 0; j < nt; ++j) {
            o.mtile_group[s_tile[ee] + j] = ee;
            o.mtile_row0[s_tile[ee] + j] = s_off[ee] + j * BM;
        }
    }
    block_sync_global();

    // phase 3: scatter every pair to its grouped row
    for (int base = 0; base < n_tiles; base += kPermWaves) {
        const int tile = base + wave;
        for (int ee = lane; ee < E; ee += kWave) mask[wave][ee] = 0ull;
        __syncthreads();
        const int t = tile * 64 + lane;
        const bool live = tile < n_tiles && t < T;
        if (live) {
            for (int k = 0; k < K; ++k)
                atomicOr(&mask[wave][topk_idx[(size_t)t * K + k]], 1ull << lane);
        }
        __syncthreads();
        if (live) {
            const unsigned long long below = (1ull << lane) - 1ull;
            for (int k = 0; k < K; ++k) {
                const size_t pk = (size_t)t * K + k;
                const int ee = topk_idx[pk];
                const int pos = o.tile_counts[(size_t)tile * E + ee] + __popcll(mask[wave][ee] & below);
                o.perm_token[pos] = t;
                o.perm_w[pos] = topk_w[pk];
                o.inv_row[pk] = pos;
            }
        }
        __syncthreads();
    }
}

hipError_t launch_permute(const float* logits, const float* pes, int32_t* topk_idx, float* topk_w,
                          int T, int K, int E, int BM, const PermuteOut& o, hipStream_t stream) {
    hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermThreads), 0, stream, logits, pes,
                       topk_idx, topk_w, T, K, E, BM, o);
    return hipGetLastError();
}

}  // namespace moe
