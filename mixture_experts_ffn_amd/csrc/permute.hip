// Expert grouping of the routed (token, slot) pairs on gfx950.
//
// Gathered expert compute (Tenstorrent bundle card, "Configurable knobs",
// GEMMA4_PREFILL_GATHERED) runs each expert only on the tokens routed to it.
// The grouping is a stable counting sort of the T*K pairs by expert (ascending
// expert, then ascending token), producing
//   counts[e], offsets[e] (exclusive prefix sum), perm_token / perm_w (token and
//   router weight of each grouped row), inv_row[t*K+k] (grouped row of a pair),
//   the list of experts with rows, and the list of BM-row tiles for the
//   grouped GEMMs.
// It is exact integer work, and deterministic: ranks come from popcounts of
// token bit masks, never from the order of atomic operations.
//
//   group_count_kernel    per tile of kRouteTile tokens: the pairs of every
//                         expert, and each pair's rank among its tile's pairs
//                         of the same expert
//   group_offsets_kernel  one workgroup: per-expert totals, offsets, active
//                         experts, GEMM M-tiles, and (in place) the first
//                         grouped row of every (tile, expert)
//   group_scatter_kernel  one thread per pair: its grouped row, and the
//                         scatter of token and weight to that row
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kOffThreads = 1024;
constexpr int kCountThreads = kRouteTile * 8;  // one thread per (token, slot), K <= 8

__global__ __launch_bounds__(kCountThreads) void group_count_kernel(
    const int32_t* __restrict__ topk_idx, int T, int K, int E, int32_t* __restrict__ tile_counts,
    int32_t* __restrict__ pair_rank) {
    __shared__ uint32_t mask[kMaxExpertsGroup];  // tokens of the tile that picked expert e
    const int tid = threadIdx.x;
    const int t0 = blockIdx.x * kRouteTile;
    const int n_pairs = min(kRouteTile, T - t0) * K;
    for (int e = tid; e < E; e += kCountThreads) mask[e] = 0u;
    __syncthreads();
    const bool live = tid < n_pairs;
    const int r = tid / K;
    const int e = live ? topk_idx[(int64_t)t0 * K + tid] : 0;
    if (live) atomicOr(&mask[e], 1u << r);
    __syncthreads();
    for (int ee = tid; ee < E; ee += kCountThreads)
        tile_counts[(int64_t)blockIdx.x * E + ee] = __popc(mask[ee]);
    if (live) pair_rank[(int64_t)t0 * K + tid] = __popc(mask[e] & ((1u << r) - 1u));
}

__global__ __launch_bounds__(kOffThreads) void group_offsets_kernel(int n_tiles, int E, int BM,
                                                                    PermuteOut o) {
    __shared__ int part[kOffThreads];
    __shared__ int s_cnt[kMaxExpertsGroup];
    __shared__ int s_off[kMaxExpertsGroup + 1];
    __shared__ int s_tile[kMaxExpertsGroup + 1];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

    // thread (e, p): expert e, the p-th chunk of tiles
    int ep = 1;
    while (ep < E) ep <<= 1;
    const int nparts = kOffThreads / ep;
    const int e = tid & (ep - 1), p = tid / ep;
    const int chunk = (n_tiles + nparts - 1) / nparts;
    const int tb = min(n_tiles, p * chunk), te = min(n_tiles, tb + chunk);
    {
        int sum = 0;
        if (e < E) {
#pragma unroll 16
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
    // first grouped row of every (tile, expert): offset + earlier tiles' counts
    if (e < E) {
        int run = s_off[e];
        for (int q = 0; q < p; ++q) run += part[q * ep + e];
#pragma unroll 16
        for (int tl = tb; tl < te; ++tl) {
            const size_t ix = (size_t)tl * E + e;
            const int cnt = o.tile_counts[ix];
            o.tile_counts[ix] = run;
            run += cnt;
        }
    }
    // tiles of BM grouped rows for the grouped GEMMs
    for (int ee = tid; ee < E; ee += kOffThreads) {
        const int nt = (s_cnt[ee] + BM - 1) / BM;
        for (int j = 0; j < nt; ++j) {
            o.mtile_group[s_tile[ee] + j] = ee;
            o.mtile_row0[s_tile[ee] + j] = s_off[ee] + j * BM;
        }
    }
    // the tile of every GEMM block (mapping of gemm_expert_blocks): block b
    // is slot local = b / kGemmXcds of XCD x = b % kGemmXcds; XCD x owns
    // M-tiles [c0, c1); its slots run over expert runs (the expert's M-tiles
    // inside the chunk), per run each N-tile with the run's M-tiles in a row
    const int m_total = s_tile[E];
    const int mchunk = (m_total + kGemmXcds - 1) / kGemmXcds;
    const int slots = (o.max_mtiles + kGemmXcds - 1) / kGemmXcds;
    for (int gi = 0; gi < 2; ++gi) {
        const int n_nt = o.n_nt[gi];
        const int n_blocks = kGemmXcds * slots * n_nt;
        for (int b = tid; b < n_blocks; b += kOffThreads) {
            const int xcd = b % kGemmXcds, local = b / kGemmXcds;
            const int c0 = xcd * mchunk, c1 = min(c0 + mchunk, m_total);
            const int mu = c0 + local / n_nt;
            int2 te = make_int2(0, -1);
            if (mu < c1) {
                int lo = 0, hi = E - 1;  // the expert g with s_tile[g] <= mu < s_tile[g + 1]
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (s_tile[mid] <= mu) lo = mid;
                    else hi = mid - 1;
                }
                const int g = lo, first = s_tile[g];
                const int r0 = max(first, c0), r1 = min(s_tile[g + 1], c1), rl = r1 - r0;
                const int ol = local - (r0 - c0) * n_nt;
                const int nt = ol / rl, mt = r0 + (ol - nt * rl);
                const int row0 = s_off[g] + (mt - first) * BM;
                const int rows = min(BM, s_off[g] + s_cnt[g] - row0);
                te = make_int2(row0, g | (rows << 9) | (nt << 18));
            }
            o.tiles[gi][b] = te;
        }
    }
}

__global__ __launch_bounds__(256) void group_scatter_kernel(const int32_t* __restrict__ topk_idx,
                                                            const float* __restrict__ topk_w,
                                                            const int32_t* __restrict__ pair_rank,
                                                            int T, int K, int E, PermuteOut o) {
    const int64_t pk = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (pk >= (int64_t)T * K) return;
    const int t = (int)(pk / K);
    const int e = topk_idx[pk];
    const int pos = o.tile_counts[(int64_t)(t / kRouteTile) * E + e] + pair_rank[pk];
    o.perm_token[pos] = t;
    o.perm_w[pos] = topk_w[pk];
    o.inv_row[pk] = pos;
}

hipError_t launch_permute(const int32_t* topk_idx, const float* topk_w, int32_t* pair_rank,
                          int T, int K, int E, int BM, const PermuteOut& o, hipStream_t stream) {
    const int n_tiles = (T + kRouteTile - 1) / kRouteTile;
    hipLaunchKernelGGL(group_count_kernel, dim3(n_tiles), dim3(kCountThreads), 0, stream, topk_idx,
                       T, K, E, o.tile_counts, pair_rank);
    hipLaunchKernelGGL(group_offsets_kernel, dim3(1), dim3(kOffThreads), 0, stream, n_tiles, E, BM, o);
    const int64_t pairs = (int64_t)T * K;
    hipLaunchKernelGGL(group_scatter_kernel, dim3((unsigned)((pairs + 255) / 256)), dim3(256), 0,
                       stream, topk_idx, topk_w, pair_rank, T, K, E, o);
    return hipGetLastError();
}

}  // namespace moe
