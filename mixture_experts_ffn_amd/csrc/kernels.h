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
// MFMA router for larger batches (fp32-exact logits via a hi/lo bf16 split of
// scale * W): per-slice partial dot products over the hidden dimension, then a
// finishing kernel (slice sum in fixed order, RMSNorm factor, bias, top-k).
struct RouterSplit {
    int slices;       // partial sums per logit
    int slice_steps;  // 64-wide K-steps per slice
};
RouterSplit router_split(int T, int H, int E);
// partial: router_split(T, H, E).slices * T * (E + 1) fp32 (logit sums, then sums of squares)
hipError_t launch_router_mfma(const uint16_t* x, const uint16_t* scale, const uint16_t* w,
                              const float* bias, const float* pes, int T, int H, int E, int K,
                              float eps, int32_t* topk_idx, float* topk_w, float* partial,
                              hipStream_t stream);
// softmax over E, top-k (ties -> lower index), renormalise, * per-expert scale
hipError_t launch_router_topk(const float* logits, const float* pes, int T, int E, int K,
                              int32_t* topk_idx, float* topk_w, hipStream_t stream);

// ---- grouping (permute.hip) ------------------------------------------------
// Tokens per grouping tile: the unit in which pairs are counted per expert.
constexpr int kRouteTile = 32;  // 32-bit token masks
constexpr int kMaxExpertsGroup = 256;
struct PermuteOut {
    int32_t* tile_counts;   // [ceil(T/kRouteTile), E]: pairs per (tile, expert) from the
                            // router; rewritten to the first grouped row of each
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
    // the tile of every block of the two expert GEMMs (0: gate/up, 1: down),
    // gemm_expert_blocks(max_mtiles, n_nt[i]) entries each: {first grouped row,
    // expert | rows << 9 | N-tile << 18}, or y = -1 for a block with no tile
    int2* tiles[2];
    int n_nt[2];
    int max_mtiles;
};
// pair_rank: [T*K] scratch (rank of each pair among its tile's pairs of the
// same expert)
hipError_t launch_permute(const int32_t* topk_idx, const float* topk_w, int32_t* pair_rank,
                          int T, int K, int E, int BM, const PermuteOut& o, hipStream_t stream);

// ---- grouped MFMA GEMMs (gemm.hip) -----------------------------------------
constexpr int kGemmBM = 256;  // rows per grouped M-tile
constexpr int kGemmBN = 256;  // output columns per N-tile (gate/up: 128 h columns)
constexpr int kGemmXcds = 8;  // block b of a GEMM runs on XCD b % 8
// N-tiles of the gate/up (h columns) and down GEMMs
inline int gemm_n_tiles_gateup(int inter) { return (inter + kGemmBN / 2 - 1) / (kGemmBN / 2); }
inline int gemm_n_tiles_down(int hidden) { return hidden / kGemmBN; }
// blocks of an expert GEMM: kGemmXcds x ceil(max_mtiles / kGemmXcds) M-tile
// slots x n_nt N-tiles. XCD x owns a contiguous chunk of the M-tiles with all
// their N-tiles, and runs them expert by expert: for each N-tile, the expert's
// M-tiles back to back, so that an N-tile's weights come from HBM once per
// expert and its other M-tiles find them in the XCD's L2.
inline int gemm_expert_blocks(int max_mtiles, int n_nt) {
    return kGemmXcds * ((max_mtiles + kGemmXcds - 1) / kGemmXcds) * n_nt;
}
constexpr int kMaxTopKGemm = 8;
struct GemmArgs {
    const uint16_t* A; int64_t lda;          // bf16 activations
    const int32_t* a_rows;                    // gather: A row of grouped row p is a_rows[p]; null = p
    const void* B; int64_t b_group_stride; int64_t ldb;  // weights [groups][rows][ldb]
    const float* b_scale; int64_t scale_group_stride;    // int8 per-row scales, null for bf16
    const float* a_scale;                     // fp8 gate/up: per-token scale of A's rows (by source row)
    int K;                                    // reduction length
    int n_out;                                // output columns
    int up_off;                               // gate/up: B row of the first up row
    const int32_t* mtile_group; const int32_t* mtile_row0; const int32_t* n_mtiles;
    const int32_t* group_end;                 // offsets[E+1] (grouped)
    int M_dense;                              // rows when not grouped
    int max_mtiles;                           // grid height
    uint16_t* C; int64_t ldc;                 // bf16 output
    float* Cf;                                // down: fp32 output instead (dense MLP)
    const float* row_w;                       // down: per-row weight of the bf16 output (null = 1)
    const int2* tiles;                        // grouped: the tile of every block (PermuteOut::tiles)
};
// gate/up + GELU of the experts, and of `dense` (bf16, may be null), in one launch
hipError_t launch_gemm_gateup(const GemmArgs& experts, const GemmArgs* dense, int wq,
                              hipStream_t stream);
// down of the experts (weighted bf16 rows) and of `dense` (fp32, may be null), in one launch
hipError_t launch_gemm_down(const GemmArgs& experts, const GemmArgs* dense, int wq,
                            hipStream_t stream);
// y[t] = dense_out[t] + sum_k rows[inv_row[t*K + k]], in k order, rounded once to bf16
hipError_t launch_combine(const float* dense_out, const uint16_t* rows, const int32_t* inv_row,
                          int T, int H, int K, uint16_t* y, hipStream_t stream);

// ---- small-batch path (decode.hip) ----------------------------------------
struct StreamArgs {
    int T, H, I, Id, K, E;
    const uint16_t* x;                        // experts input
    const uint16_t* xr;                       // router input
    const uint16_t* xd;                       // dense MLP input
    // E4M3 experts: x quantised per token (half carriers of value * 2^-8) and its per-token scales
    uint16_t* xq; float* x_scale;  // written by decode_front's first workgroups
    // the layer's pre-norms, folded into decode_front (null pre_src: none): the
    // residual stream, the dense and MoE branches' gains (either may be null),
    // eps, and the branch inputs they write (x_d = bf16(N_gd(h)), x_m = bf16(N_gm(h)))
    const uint16_t* pre_src; const uint16_t* pre_gd; const uint16_t* pre_gm; float pre_eps;
    uint16_t* pre_xd; uint16_t* pre_xm;
    // experts
    const void* gu; const float* gu_scale;   // [E][2I][H]
    const void* dw; const float* dw_scale;   // [E][H][I]
    int32_t* counts; int32_t* offsets; int32_t* active; int32_t* n_active;
    int32_t* perm_token; float* perm_w; int32_t* inv_row;
    const float* topk_w;                      // [T][K] router weights (K2 writes them)
    int max_active;                           // 0 = no expert items
    // dense
    int with_dense;                           // the launch carries the dense MLP's items
    int front_dense;                          // dense gate/up items in K1 (else in K2)
    const uint16_t* dgu; const uint16_t* ddw;
    // intermediates and output
    uint16_t* h;    // [T*K][I]
    float* h_scale; // E4M3 experts: scale of each row of h (grouped order), times 2^16
    uint16_t* hd;   // [T][Id]
    uint16_t* y;    // [T][H]
    // fp32 partial outputs of K4: expert rows [T*K][H] (grouped order), dense [T][H]
    float* part; float* dpart;
    // fp32 partial sums of the dense gate/up, K split: [kFrontSplit][T][2 Id] (gate, then up)
    float* dgu_part;
    // fp32 partial sums of the experts' gate/up, the two halves of K: [2][T*K][2 I]
    float* hpart;
};
// workgroups sharing the K range of one router or dense gate/up item in K1
constexpr int kFrontSplit = 4;
// K1: router partial logits lpart [kFrontSplit][T][E] and sums of squares of x
// ss_part [kFrontSplit][T] (if wr != null), beside the dense gate/up partial
// sums -> dgu_part (if a.with_dense and a.front_dense)
hipError_t launch_decode_front(const StreamArgs& a, const uint16_t* scale, const uint16_t* wr, float* lpart,
                               float* ss_part, hipStream_t stream);
// K2: logits from the partial sums, top-k and grouping (one workgroup, T <=
// MOE_STREAM_MAX_TOKENS; none if lpart == null) beside the dense gate/up
// partial sums (-> dgu_part, if a.with_dense and not a.front_dense)
hipError_t launch_decode_route(const StreamArgs& a, const float* lpart, const float* ss_part, const float* bias,
                               const float* pes, float eps, int32_t* topk_idx, float* topk_w,
                               hipStream_t stream);
// K3: the dense gate/up finish (dgu_part -> hd, if a.with_dense), then the gate/up of the
// touched experts -> fp32 partial sums of the two halves of K (hpart)
hipError_t launch_decode_experts_gateup(const StreamArgs& a, int wq, hipStream_t stream);
// K4: h from hpart, down of the touched experts and of the dense MLP -> fp32 partial rows
hipError_t launch_decode_down(const StreamArgs& a, int wq, hipStream_t stream);
// E4M3 experts: h of every routed pair formed and quantised per row (a.h, a.h_scale)
hipError_t launch_decode_hquant(const StreamArgs& a, hipStream_t stream);
// K5: y = dense + sum_k w_k * expert rows (k order) -> bf16
hipError_t launch_decode_combine(const StreamArgs& a, hipStream_t stream);

// ---- int8 quantiser (quant.hip) -------------------------------------------
// row-major [rows, cols] -> tiled layout (16 x 64 tiles); rows % 16 == 0, cols % 64 == 0
hipError_t launch_tile_weights(const void* src, int64_t rows, int cols, bool int8, void* dst,
                               hipStream_t stream);
hipError_t launch_quantize_int8(const uint16_t* w, int64_t rows, int cols, int8_t* q, float* scale,
                                hipStream_t stream);
// E4M3 per row: weights -> codes + scales
hipError_t launch_quantize_fp8(const uint16_t* w, int64_t rows, int cols, uint8_t* q, float* scale,
                               hipStream_t stream);
// activations -> per-row E4M3 code bytes for the E4M3 MFMAs: rows of ldq bytes
// (ldq a multiple of 128, >= cols, the tail zero), + scale, + mul_out = mul_in * scale
hipError_t launch_act_quant_fp8_bytes(const uint16_t* x, int64_t rows, int cols, uint8_t* q, int ldq, float* scale,
                                      const float* mul_in, float* mul_out, hipStream_t stream);
// row length in bytes of E4M3 activation codes of `cols` values (a whole number of 128-code K-steps)
inline int fp8_row_bytes(int cols) { return (cols + 127) / 128 * 128; }

// ---- the layer's feed-forward norms around the block (ffn.hip) ----------------
// x_d = bf16(N_gd(h)), x_m = bf16(N_gm(h)) per token (only those whose gain is given)
hipError_t launch_ffn_prenorm(const uint16_t* h, int T, int H, const uint16_t* gd, const uint16_t* gm, float eps,
                              uint16_t* xd, uint16_t* xm, hipStream_t stream);
// out = h + N_gp(N_gpd(dense) + N_gpm(moe)), moe = sum_k rows[inv_row[t K + k]] in k order
// (f32_rows: fp32 rows times topk_w; else bf16 rows already weighted); absent gain: no norm
hipError_t launch_ffn_post(const uint16_t* h, const float* dense, const void* rows, bool f32_rows,
                           const int32_t* inv_row, const float* topk_w, int T, int H, int K,
                           const uint16_t* gpd, const uint16_t* gpm, const uint16_t* gp, float eps, uint16_t* out,
                           hipStream_t stream);

}  // namespace moe
