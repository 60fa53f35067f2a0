/*
 * moe.h -- C ABI of libmoe_ffn.so, the MI355X (gfx950) hybrid MoE FFN block.
 *
 * The block is the feed-forward part of a Gemma-4 26B-A4B layer: a 128-expert
 * top-8 mixture of GeGLU experts running in parallel with a shared dense MLP.
 * Pages that define it (titles as printed on them):
 *   [INF2] "Gemma-4 26B-A4B (MoE) on AWS Inferentia2 -- Tensor-Parallel (TP=8)"
 *          sections "The architecture (a dual-path FFN)", "How it works (the recipe)"
 *   [INT8] "Gemma-4 26B-A4B (MoE, int8 experts) on AWS Inferentia2 -- TP=8"
 *          intro and "How it works"
 *   [TT]   "Gemma-4-26B-A4B-it -- Tenstorrent Blackhole (vLLM bundle)"
 *          "Configurable knobs" (gathered expert prefill)
 *   [ONNX] "Gemma-4 26B-A4B-it -- ONNX MoE text decoder (fp16, CUDA) with
 *          canonical inference metadata", table "Truthful graph contracts"
 *          (rows "Mixture of Experts", "MoE topology", "Router") and
 *          "MoE dispatch: why this export uses the vectorized unfused path"
 *   [VLLM] "Gemma 4 26B-A4B IT" (vLLM recipe), its "variants" list, fp8 entry
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is a DEVICE pointer owned by the caller, contiguous,
 *   row-major and 16-byte aligned. bf16 tensors hold bfloat16 bit patterns.
 * - `ws` is caller-owned device scratch of at least moe_workspace_bytes(d, T)
 *   bytes, 256-byte aligned. Its contents on entry do not matter; calls that
 *   share one workspace must not overlap in time.
 * - Work is enqueued on `stream` (0 = the null stream) and the call returns
 *   without waiting for it; there is no host synchronisation, no allocation
 *   and no global device state. Device faults surface at the caller's next
 *   synchronisation.
 * - Every call checks its arguments before it launches anything. On error it
 *   returns a negative status, launches nothing and leaves a message for
 *   moe_last_error(); there is no fallback to another implementation.
 * - T == 0 is a valid empty batch: the call returns MOE_OK and launches nothing;
 *   the activation, output and workspace pointers may then be NULL.
 *
 * Shape limits: hidden % 256 == 0; expert_inter % 64 == 0; dense_inter % 64 == 0;
 * 1 <= top_k <= 8; top_k <= num_experts <= 256; 0 <= T <= MOE_MAX_TOKENS.
 */
#ifndef MOE_FFN_H
#define MOE_FFN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define MOE_OK               0
#define MOE_ERR_NULL        -1  /* a required pointer is NULL */
#define MOE_ERR_SHAPE       -2  /* T < 0 or > MOE_MAX_TOKENS, or a dimension breaks the limits above */
#define MOE_ERR_UNSUPPORTED -3  /* top_k > 8, num_experts > 256, unknown dtype or path */
#define MOE_ERR_WORKSPACE   -4  /* ws_bytes smaller than moe_workspace_bytes() */
#define MOE_ERR_HIP         -5  /* a HIP launch or copy failed; the message names it */
#define MOE_ERR_ALIGN       -6  /* a tensor is not 16-byte aligned, or ws not 256-byte aligned */

#define MOE_MAX_TOKENS   (1 << 22)
#define MOE_MAX_EXPERTS  256
#define MOE_MAX_TOPK     8

/* expert weight storage */
#define MOE_DTYPE_BF16 0
#define MOE_DTYPE_INT8 1  /* [INT8]: per-output-channel symmetric int8 + fp32 scale */
#define MOE_DTYPE_FP8  2  /* [VLLM] fp8 variant: E4M3 codes + fp32 per-output-channel scale; the
                             experts' inputs are quantised per token inside the block */

/* how moe_block computes the routed experts */
#define MOE_PATH_AUTO    0  /* streaming when T <= the streaming limit, else grouped */
#define MOE_PATH_STREAM  1  /* weight-streaming kernels, each weight row read once (small T) */
#define MOE_PATH_GROUPED 2  /* grouped MFMA GEMMs over the gathered (token, expert) rows */

/* Largest T the streaming path accepts (its per-block staging is sized for it). */
#define MOE_STREAM_MAX_TOKENS 64

/* Storage of the expert and dense weight matrices (moe_weights.layout).
 * MOE_LAYOUT_TILED is the one the block kernels read: a row-major matrix
 * W [rows, cols] (rows % 16 == 0, cols % 64 == 0) is cut into 16-row x
 * 64-column tiles, stored tile-row-major (tile (i, j) at tile index
 * i * cols/64 + j); inside a tile, element (r, c) sits at lane
 * 16 * (c / 16) + r, position c % 16 of that lane's 16 values, and
 *   bf16: tile = 2048 bytes, byte (c % 16 / 8) * 1024 + lane * 16 + (c % 8) * 2
 *   int8: tile = 1024 bytes, byte lane * 16 + c % 16.
 * So each 16-byte piece a lane of a 64-lane wavefront needs for one 16x16x32
 * MFMA operand (or one 16-row GEMV step) is one piece of a contiguous 1 KB
 * run, and a 16-row block of W is one contiguous stream. A tiled matrix has
 * the size of the row-major one, and an expert's matrix starts where it would
 * in the row-major [E, rows, cols] array. moe_tile_weights produces it. */
#define MOE_LAYOUT_ROWS  0  /* row-major: not accepted by moe_block / dense_mlp */
#define MOE_LAYOUT_TILED 1

/* Block dimensions. [INF2] "The architecture (a dual-path FFN)": hidden 2816,
 * 128 experts, top 8, expert intermediate 704, dense intermediate 2112.
 * rms_eps: the router's RMSNorm epsilon (added to mean(x^2) inside the root). */
typedef struct moe_dims {
    int32_t hidden;        /* H  */
    int32_t num_experts;   /* E  */
    int32_t top_k;         /* K  */
    int32_t expert_inter;  /* I  */
    int32_t dense_inter;   /* Id */
    float   rms_eps;
} moe_dims;

/* One layer's weights (all device pointers). Router tensors are row-major;
 * the four expert / dense matrices are in the layout named by `layout`.
 * Router, [ONNX] row "Router": logits = (x / rms(x)) * router_scale * H^-0.5 @ router_w^T
 *   (+ logit_bias), softmax in fp32, top-k, renormalise, * per_expert_scale.
 * Experts, [INF2] "How it works (the recipe)" and [ONNX] row "Mixture of Experts":
 *   out = down @ (gelu_tanh(gate @ x) * (up @ x)); gate_up rows [0,I) are gate,
 *   rows [I,2I) are up. Dense MLP ([ONNX] row "MoE topology") has the same form
 *   with Id. */
typedef struct moe_weights {
    const void*  router_scale;      /* [H]      bf16 */
    const void*  router_w;          /* [E, H]   bf16 */
    const float* per_expert_scale;  /* [E]      fp32 */
    const float* logit_bias;        /* [E]      fp32, or NULL for none */
    const void*  expert_gate_up;    /* [E, 2I, H]  bf16, or int8 / E4M3 codes (1 byte) per expert_dtype */
    const void*  expert_down;       /* [E, H, I]   bf16, or int8 */
    int32_t      expert_dtype;      /* MOE_DTYPE_* */
    const float* gate_up_scale;     /* [E, 2I] fp32 per-row scales (INT8 and FP8; else ignored) */
    const float* down_scale;        /* [E, H]  fp32 per-row scales (INT8 and FP8; else ignored) */
    const void*  dense_gate_up;     /* [2Id, H] bf16 */
    const void*  dense_down;        /* [H, Id]  bf16 */
    int32_t      layout;            /* MOE_LAYOUT_TILED (MOE_LAYOUT_ROWS is rejected) */
} moe_weights;

#define MOE_MAX_STAGES 8

/* Optional parity / timing hooks for moe_block (pass NULL for none).
 * Every output pointer is a device pointer or NULL (then it is skipped); the
 * library copies into them on `stream` after the block has been computed. */
typedef struct moe_debug {
    int32_t  path;             /* in:  MOE_PATH_* */
    int32_t* topk_idx;         /* out: [T, K] selected experts, descending logit, ties -> lower index */
    float*   topk_w;           /* out: [T, K] renormalised weights times per_expert_scale */
    int32_t* counts;           /* out: [E]    rows per expert */
    int32_t* offsets;          /* out: [E+1]  exclusive prefix sum of counts */
    int32_t* perm_token;       /* out: [T*K]  token of each grouped row (ascending expert, then token) */
    int32_t* inv_row;          /* out: [T*K]  grouped row of pair (t, k), at index t*K + k */
    hipEvent_t stage_event[MOE_MAX_STAGES + 1]; /* in: if non-NULL, event i is recorded on `stream`
                                   before stage i and event n_stages after the last one */
    int32_t  path_taken;       /* out (host): the path used */
    int32_t  n_stages;         /* out (host): stages launched; a stage is one to three kernel launches */
    const char* stage_name[MOE_MAX_STAGES]; /* out (host): kernel of each stage (static strings) */
} moe_debug;

/* Exact device bytes moe_block, moe_route and dense_mlp need at this T
 * (router logits, routing, grouping tables, intermediates). 0 if the
 * dimensions are invalid (moe_last_error() says why). */
size_t moe_workspace_bytes(const moe_dims* d, int32_t T);

/* Router alone. [ONNX] "Truthful graph contracts", row "Router".
 * x [T, H] bf16 -> topk_idx [T, K] int32 (descending logit; equal logits go to
 * the lower expert index), topk_w [T, K] fp32 (renormalised softmax weights of
 * the selected experts times per_expert_scale). The router runs in fp32
 * throughout: RMSNorm, scale, logits, softmax. */
int moe_route(const moe_dims* d, const moe_weights* w, const void* x, int32_t T,
              int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes, hipStream_t stream);

/* The whole block. y [T, H] bf16 = dense(x) + sum_k topk_w[t,k] * expert_{topk_idx[t,k]}(x_t)
 * ([ONNX] row "MoE topology": dense MLP in parallel with the MoE; [INF2] "How it
 * works": sparse top-k, equal to all-experts-dense with zero weight on unselected
 * experts). Only the routed (token, expert) pairs are computed ([TT] "Configurable
 * knobs", gathered expert prefill). GEMMs accumulate in fp32 ([ONNX] "MoE
 * dispatch": fp16 accumulation loses accuracy at hidden 2816); the GeGLU
 * intermediates are rounded to bf16 before the down projections. The result is
 * deterministic: no floating-point atomics, fixed summation order over k.
 * dbg may be NULL. */
int moe_block(const moe_dims* d, const moe_weights* w, const void* x, int32_t T, void* y,
              moe_debug* dbg, void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_block without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). Its kernels use the library's own scratch array, of
 * MOE_NOALLOC_SCRATCH_BYTES per device, which each device the library runs on
 * holds from the library's load until the process ends; nothing is allocated
 * or freed on any call. The array's device address is looked up once per
 * device, on the first call made with that device current. Arguments, result,
 * path choice and errors are those of moe_block, and so is the output, bit for
 * bit. A batch whose workspace (moe_workspace_bytes) exceeds the array is
 * refused with MOE_ERR_WORKSPACE before anything is launched: at the real
 * shape that admits every decode-sized batch (T <= 64) and grouped batches of
 * up to 374 tokens. Every call on one device shares its array and leaves its
 * intermediates there (no kernel relies on what an earlier call left): calls
 * that overlap on one device, from several streams or threads, race and must
 * be serialised by the caller. */
#define MOE_NOALLOC_SCRATCH_BYTES (32 << 20)
int moe_block_noalloc(const moe_dims* d, const moe_weights* w, const void* x, int32_t T, void* y,
                      moe_debug* dbg, hipStream_t stream);

/* The shared dense MLP alone ([ONNX] row "MoE topology"): y [T, H] bf16 =
 * dense_down @ (gelu_tanh(gate @ x) * (up @ x)), with dense_gate_up [2Id, H]
 * (gate rows first) and dense_down [H, Id], all bf16 and in MOE_LAYOUT_TILED. Uses d->hidden and
 * d->dense_inter; the expert fields of d must still be valid. */
int dense_mlp(const moe_dims* d, const void* dense_gate_up, const void* dense_down,
              const void* x, int32_t T, void* y, void* ws, size_t ws_bytes, hipStream_t stream);

/* Gains of the feed-forward layernorms around the block (moe_ffn_layer). Each
 * is a device pointer to H bf16 values (16-byte aligned), or NULL: no norm at
 * that position. N_g(v) = v / sqrt(mean(v^2) + eps) * g, per token, in fp32. */
typedef struct moe_ffn_norms {
    const void* pre_dense;   /* dense MLP branch input */
    const void* pre_moe;     /* MoE branch input (the experts; the router reads h) */
    const void* post_dense;  /* dense MLP branch output */
    const void* post_moe;    /* MoE branch output */
    const void* post;        /* their sum, before the residual */
    float eps;
} moe_ffn_norms;

/* The layer's feed-forward part around the block ([INF2] "The architecture (a
 * dual-path FFN)": the dense MLP and the MoE run in parallel and pass through
 * four feed-forward layernorms; [ONNX] "Truthful graph contracts", row "MoE
 * topology": post_ff_norm(dense + moe) + residual):
 *   out = h + N_post(N_post_dense(dense(x_d)) + N_post_moe(moe(x_m))),
 *   x_d = bf16(N_pre_dense(h)), x_m = bf16(N_pre_moe(h)),
 * dense and moe as in moe_block (the experts on x_m, the dense MLP on x_d), the
 * router on h itself: its own first step is a scale-free RMSNorm ([ONNX] row
 * "Router"), the norm of a router that reads the un-normalised stream. The
 * branch outputs stay fp32 through the post-norms and the residual add, and
 * out is rounded once to bf16. h, out [T, H] bf16 (out may not alias h); n as
 * above (NULL: every norm absent, the residual kept); ws as for moe_block
 * (moe_ffn_workspace_bytes: its size); dbg as for moe_block, its routing being
 * that of h. hidden <= 16384. Errors as for moe_block, plus
 * MOE_ERR_ALIGN for a misaligned gain and MOE_ERR_UNSUPPORTED for a larger
 * hidden size. */
size_t moe_ffn_workspace_bytes(const moe_dims* d, int32_t T);
int moe_ffn_layer(const moe_dims* d, const moe_weights* w, const moe_ffn_norms* n, const void* h,
                  int32_t T, void* out, moe_debug* dbg, void* ws, size_t ws_bytes, hipStream_t stream);

/* Chunked prefill ([TT] "Configurable knobs": a long prompt is prefilled in
 * bounded token chunks, 16384 by default, the size snapped to a multiple of the
 * 1024-token sliding window and capped at 32768, so that peak prefill memory
 * does not grow with the prompt).
 * moe_prefill_chunk_tokens: the chunk size used for a requested one: <= 0 gives
 * 16384; otherwise rounded down to a multiple of 1024, at least 1024 and at
 * most 32768. Host arithmetic only.
 * moe_prefill_workspace_bytes: workspace for chunks of that size (the layer's,
 * which covers the block's), 0 on invalid dims.
 * moe_prefill_chunked: runs consecutive chunks of h [T, H] (the last one
 * ragged) through the block on `stream`, one after another, reusing ws.
 * n == NULL: out = moe_block(h) per chunk; n != NULL: out = moe_ffn_layer(h, n)
 * per chunk. Each token's result depends only on that token, so the output
 * equals the per-chunk calls bit for bit; each chunk takes the path moe_block
 * would take at its size. out [T, H] bf16, may not alias h. ws must hold
 * moe_prefill_workspace_bytes(d, chunk) bytes for chunk =
 * moe_prefill_chunk_tokens(chunk_tokens) (less when T is smaller: the
 * workspace of min(T, chunk) tokens). Errors as for moe_ffn_layer. */
int32_t moe_prefill_chunk_tokens(int32_t chunk_tokens);
size_t moe_prefill_workspace_bytes(const moe_dims* d, int32_t chunk_tokens);
int moe_prefill_chunked(const moe_dims* d, const moe_weights* w, const moe_ffn_norms* n, const void* h,
                        int32_t T, int32_t chunk_tokens, void* out, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/* Per-row symmetric int8 quantisation of a bf16 matrix [rows, cols], as the
 * int8 build quantises the fused expert weights when it loads them ([INT8]
 * "How it works"): scale[r] = max_c |w[r,c]| / 127 (fp32), q[r,c] =
 * round-half-even(w[r,c] / scale[r]) clamped to [-127, 127]; an all-zero row
 * gets scale 0 and q 0. cols % 8 == 0, rows >= 0. Writes q [rows, cols] int8
 * and scale [rows] fp32. */
int moe_quantize_int8(const void* w_bf16, int64_t rows, int32_t cols, int8_t* q, float* scale,
                      hipStream_t stream);

/* Per-row E4M3 quantisation of a bf16 matrix [rows, cols] ([VLLM] "variants",
 * fp8: E4M3 weights with dynamic per-token activation quantisation; the E4M3
 * format is the OCP one without infinities: bias 7, largest finite 448):
 * scale[r] = max_c |w[r,c]| / 448 (fp32), q[r,c] = the E4M3 code nearest to
 * w[r,c] / scale[r] (fp32 division), ties to the even code; an all-zero row
 * gets scale 0 and codes 0. cols % 8 == 0, rows >= 0. Writes q [rows, cols]
 * (one byte each) and scale [rows] fp32. With expert_dtype = MOE_DTYPE_FP8 the
 * block quantises the experts' inputs the same way, per token: x before the
 * gate/up projection, h (rounded to bf16) before the down projection. */
int moe_quantize_fp8(const void* w_bf16, int64_t rows, int32_t cols, uint8_t* q, float* scale,
                     hipStream_t stream);

/* Re-lays a row-major matrix into MOE_LAYOUT_TILED (see above): src [rows, cols]
 * of dtype MOE_DTYPE_BF16, MOE_DTYPE_INT8 or MOE_DTYPE_FP8 -> dst, same size, a different
 * buffer. An [E, rows, cols] stack of expert matrices is one matrix of E * rows
 * rows. rows % 16 == 0, cols % 64 == 0, rows >= 0. Pure data movement: the
 * values are the same bits. */
int moe_tile_weights(const void* src, int64_t rows, int32_t cols, int32_t dtype, void* dst,
                     hipStream_t stream);

/* Message for the last non-zero status returned on this thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_FFN_H */
