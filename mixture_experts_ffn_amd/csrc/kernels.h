// Host-side launchers of the MoE FFN kernels (implemented in the .hip files).
// Every launcher enqueues on `stream` and returns hipGetLastError().
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---- router (router.hip) -------------------------------------------------
// logits[t, e] = rms(x_t)^-1 * H^-0.5 * sum_h x[t,h] s[h] W[e,h] (+ bias[e]), fp32.
hipError_t launch_router_logits(const uint16_t* x, const uint16_t* scale, const uint16_t* w,
                                const float* bias, int T, int H, int E, float eps,
                                float* logits, hipStream_t stream);
// softmax over E, top-k (ties -> lower index), renormalise, * per-expert scale
hipError_t launch_router_topk(const float* logits, const float* pes, int T, int E, int K,
                              int32_t* topk_idx, float* topk_w, hipStream_t stream);

// ---- grouping (permute.hip) ------------------------------------------------
struct PermuteOut {
    int32_t* tile_counts;   // [ceil(T/64), E] scratch
    int32_t* counts;        // [E]
    int32_t* offsets;       // [E+1]
    int32_t* perm_token;    // [T*K]
    float*   perm_w;        // [T*K]
    int32_t* inv_row;       // [T*K]
    int32_t* active;        // [E] experts with rows, ascending
    int32_t* n_active;      // [1]
    int32_t* mtile_group;   // [max m-tiles] expert of each BM-row tile
    int32_t* mtile_row0;    // [max m-tiles] first grouped row of each tile
    int32_t* n_mtiles;      // [1]
};
// If `logits` is non-null the kernel first runs the top-k for all T tokens
// (small T) and writes topk_idx / topk_w itself.
hipError_t launch_permute(const float* logits, const float* pes, int32_t* topk_idx, float* topk_w,
                          int T, int K, int E, int BM, const PermuteOut& o, hipStream_t stream);

// ---- grouped MFMA GEMMs (gemm.hip) -----------------------------------------
constexpr int kGemmBM = 128;
struct GemmArgs {
    const uint16_t* A; int64_t lda;          // bf16 activations
    const int32_t* a_rows;                    // gather: A row of grouped row p is a_rows[p]; null = p
    const void* B; int64_t b_group_stride; int64_t ldb;  // weights [groups][rows][ldb]
    const float* b_scale; int64_t scale_group_stride;    // int8 per-row scales, null for bf16
    int K;                                    // reduction length
    int n_out;                                // output columns
    int up_off;                               // gate/up: B row of the first up row
    const int32_t* mtile_group; const int32_t* mtile_row0; const int32_t* n_mtiles;
    const int32_t* group_end;                 // offsets[E+1] (grouped)
    int M_dense;                              // rows when not grouped
    int max_mtiles;                           // grid height
    uint16_t* C; int64_t ldc;                 // bf16 output
    const float* row_w;                       // down: per-row weight
    const uint16_t* comb; const int32_t* inv_row; int topk;  // combine: rows added to y
};
hipError_t launch_gemm_gateup(const GemmArgs& a, bool int8, hipStream_t stream);
hipError_t launch_gemm_down(const GemmArgs& a, bool int8, hipStream_t stream);
hipError_t launch_gemm_combine(const GemmArgs& a, hipStream_t stream);

// ---- weight-streaming kernels for small T (stream.hip) --------------------
struct StreamArgs {
    int T, H, I, Id, K, E;
    const uint16_t* x;
    // experts
    const void* gu; const float* gu_scale;   // [E][2I][H]
    const void* dw; const float* dw_scale;   // [E][H][I]
    const int32_t* active; const int32_t* n_active; const int32_t* offsets;
    const int32_t* perm_token; const float* perm_w; const int32_t* inv_row;
    int max_active;                           // 0 = dense only
    // dense
    const uint16_t* dgu; const uint16_t* ddw;
    // intermediates and output
    uint16_t* h;    // [T*K][I]
    uint16_t* hd;   // [T][Id]
    uint16_t* y;    // [T][H]
};
hipError_t launch_stream_gateup(const StreamArgs& a, bool int8, hipStream_t stream);
hipError_t launch_stream_down(const StreamArgs& a, bool int8, hipStream_t stream);

// ---- int8 quantiser (quant.hip) -------------------------------------------
hipError_t launch_quantize_int8(const uint16_t* w, int64_t rows, int cols, int8_t* q, float* scale,
                                hipStream_t stream);

}  // namespace moe
