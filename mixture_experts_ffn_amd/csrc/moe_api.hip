// Host side of libmoe_ffn.so: argument checks, workspace carving, path
// selection and kernel launches for the C ABI declared in include/moe.h.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/moe.h"
#include "kernels.h"

// The workspace of moe_block_noalloc: a fixed array that the code object
// brings to every device the library runs on (each device holds its own copy,
// at its own address, until the process ends). Host code never uses this
// name as a device address: it reads each device's address once with
// hipGetSymbolAddress and passes that to the kernels.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

#define HIP_TRY(expr, what)                                                                     \
    do {                                                                                        \
        hipError_t e_ = (expr);                                                                 \
        if (e_ != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e_)); \
    } while (0)

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t up256(size_t b) { return (b + 255) & ~size_t(255); }

// moe_route: above this many tokens the MFMA router (fused with the top-k)
// runs; below it, the per-expert dot-product router and a separate top-k,
// which spread a small batch over more workgroups.
constexpr int kRouterMfmaMinT = 64;
// the small-batch router stages 8 token rows in LDS (16 * hidden bytes); wider
// rows take the MFMA router, whose LDS does not grow with hidden
constexpr int kRouterLogitsMaxHidden = 4096;
constexpr int kFfnMaxHidden = 16384;  // the norm kernels hold a row in registers
// chunked prefill: default and largest chunk, and the sliding window the size is a multiple of
constexpr int32_t kPrefillChunkDefault = 16384;
constexpr int32_t kPrefillChunkMax = 32768;
constexpr int32_t kSlidingWindow = 1024;

// Workspace layout at a given T (byte offsets into ws).
struct Layout {
    size_t logits, partial, topk_idx, topk_w, pair_rank, tile_counts, counts, offsets, active, n_active;
    size_t perm_token, perm_w, inv_row, mtile_group, mtile_row0, n_mtiles, gemm_tiles[2], h, hd, rows;
    size_t dout, part, dpart, dgu_part, lpart, ss_part, hpart, xq, xscale, hq, hscale, wrow, total;
    int max_mtiles;
};

Layout make_layout(const moe_dims& d, int64_t T) {
    Layout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += up256(bytes);
        return o;
    };
    const int64_t E = d.num_experts, K = d.top_k, TK = T * K;
    const int64_t n_tiles = (T + moe::kRouteTile - 1) / moe::kRouteTile;
    const int64_t BM = moe::kGemmBM;
    L.max_mtiles = (int)((TK + BM - 1) / BM + (E < TK ? E : TK));
    // fp32 logits: only moe_route's small-batch router stages them
    L.logits = take((T <= kRouterMfmaMinT && d.hidden <= kRouterLogitsMaxHidden ? T : 0) * E * 4);
    // MFMA router's partial sums and sums of squares (every T: the grouped path uses it at any size)
    L.partial = take(T > 0 ? (size_t)moe::router_split((int)T, d.hidden, (int)E).slices * T * (E + 1) * 4 : 0);
    L.topk_idx = take(TK * 4);
    L.topk_w = take(TK * 4);
    L.pair_rank = take(TK * 4);
    L.tile_counts = take(n_tiles * E * 4);
    L.counts = take(E * 4);
    L.offsets = take((E + 1) * 4);
    L.active = take(E * 4);
    L.n_active = take(4);
    L.perm_token = take(TK * 4);
    L.perm_w = take(TK * 4);
    L.inv_row = take(TK * 4);
    L.mtile_group = take((size_t)L.max_mtiles * 4);
    L.mtile_row0 = take((size_t)L.max_mtiles * 4);
    L.n_mtiles = take(4);
    L.gemm_tiles[0] = take((size_t)moe::gemm_expert_blocks(L.max_mtiles, moe::gemm_n_tiles_gateup(d.expert_inter)) * 8);
    L.gemm_tiles[1] = take((size_t)moe::gemm_expert_blocks(L.max_mtiles, moe::gemm_n_tiles_down(d.hidden)) * 8);
    L.h = take(TK * d.expert_inter * 2);
    L.hd = take(T * d.dense_inter * 2);
    L.rows = take(TK * d.hidden * 2);
    L.dout = take(T * d.hidden * 4);  // dense MLP output (fp32) before the combine
    // streaming-path scratch (only T <= MOE_STREAM_MAX_TOKENS uses it)
    const int64_t Ts = T <= MOE_STREAM_MAX_TOKENS ? T : 0;
    L.part = take(Ts * K * d.hidden * 4);
    L.dpart = take(Ts * d.hidden * 4);
    L.dgu_part = take(Ts * moe::kFrontSplit * 2 * d.dense_inter * 4);
    L.lpart = take(Ts * moe::kFrontSplit * E * 4);
    L.ss_part = take(Ts * moe::kFrontSplit * 4);
    L.hpart = take(2 * Ts * K * 2 * d.expert_inter * 4);
    // E4M3 experts: x quantised per token (half carriers on the streaming path,
    // code bytes on the grouped one) and its scales; h's codes (grouped path,
    // rows padded to whole 128-code K-steps), per-row scales and the down
    // projection's row factors (router weight x scale, x 2^16 for carriers)
    L.xq = take(T * d.hidden * 2);
    L.xscale = take(T * 4);
    L.hq = take(TK * moe::fp8_row_bytes(d.expert_inter));
    L.hscale = take(TK * 4);
    L.wrow = take(TK * 4);
    L.total = off;
    return L;
}

int check_dims(const moe_dims* d) {
    if (!d) return fail(MOE_ERR_NULL, "dims is NULL");
    if (d->top_k > MOE_MAX_TOPK)
        return fail(MOE_ERR_UNSUPPORTED, "top_k=%d > %d", d->top_k, MOE_MAX_TOPK);
    if (d->num_experts > MOE_MAX_EXPERTS)
        return fail(MOE_ERR_UNSUPPORTED, "num_experts=%d > %d", d->num_experts, MOE_MAX_EXPERTS);
    if (d->hidden <= 0 || d->hidden % 256)
        return fail(MOE_ERR_SHAPE, "hidden=%d must be a positive multiple of 256", d->hidden);
    if (d->expert_inter <= 0 || d->expert_inter % 64)
        return fail(MOE_ERR_SHAPE, "expert_inter=%d must be a positive multiple of 64", d->expert_inter);
    if (d->dense_inter <= 0 || d->dense_inter % 64)
        return fail(MOE_ERR_SHAPE, "dense_inter=%d must be a positive multiple of 64", d->dense_inter);
    if (d->top_k < 1 || d->num_experts < d->top_k)
        return fail(MOE_ERR_SHAPE, "need 1 <= top_k (%d) <= num_experts (%d)", d->top_k, d->num_experts);
    if (!(d->rms_eps >= 0.f) || d->rms_eps > 1.f)
        return fail(MOE_ERR_SHAPE, "rms_eps=%g must be in [0, 1]", (double)d->rms_eps);
    return MOE_OK;
}

int check_tiled(const moe_weights* w) {
    if (w->layout != MOE_LAYOUT_TILED)
        return fail(MOE_ERR_UNSUPPORTED, "layout=%d: expert and dense weights must be MOE_LAYOUT_TILED "
                    "(see moe_tile_weights)", w->layout);
    return MOE_OK;
}

int check_T(int32_t T) {
    if (T < 0 || T > MOE_MAX_TOKENS) return fail(MOE_ERR_SHAPE, "T=%d outside [0, %d]", T, MOE_MAX_TOKENS);
    return MOE_OK;
}

int check_ws(const moe_dims* d, int32_t T, void* ws, size_t ws_bytes) {
    if (!ws) return fail(MOE_ERR_NULL, "workspace is NULL");
    if (!aligned(ws, 256)) return fail(MOE_ERR_ALIGN, "workspace must be 256-byte aligned");
    const size_t need = make_layout(*d, T).total;
    if (ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes < %zu needed at T=%d", ws_bytes, need, T);
    return MOE_OK;
}

#define CHECK_PTR(p, name, al)                                                       \
    do {                                                                             \
        if (!(p)) return fail(MOE_ERR_NULL, "%s is NULL", name);                     \
        if (!aligned((p), (al))) return fail(MOE_ERR_ALIGN, "%s is not %d-byte aligned", name, (al)); \
    } while (0)

int check_weights(const moe_weights* w) {
    if (!w) return fail(MOE_ERR_NULL, "weights is NULL");
    CHECK_PTR(w->router_scale, "router_scale", 16);
    CHECK_PTR(w->router_w, "router_w", 16);
    CHECK_PTR(w->per_expert_scale, "per_expert_scale", 4);
    if (w->logit_bias && !aligned(w->logit_bias, 4)) return fail(MOE_ERR_ALIGN, "logit_bias misaligned");
    CHECK_PTR(w->expert_gate_up, "expert_gate_up", 16);
    CHECK_PTR(w->expert_down, "expert_down", 16);
    if (w->expert_dtype != MOE_DTYPE_BF16 && w->expert_dtype != MOE_DTYPE_INT8 && w->expert_dtype != MOE_DTYPE_FP8)
        return fail(MOE_ERR_UNSUPPORTED, "expert_dtype=%d", w->expert_dtype);
    if (w->expert_dtype != MOE_DTYPE_BF16) {
        CHECK_PTR(w->gate_up_scale, "gate_up_scale", 4);
        CHECK_PTR(w->down_scale, "down_scale", 4);
    }
    CHECK_PTR(w->dense_gate_up, "dense_gate_up", 16);
    CHECK_PTR(w->dense_down, "dense_down", 16);
    return MOE_OK;
}

// Largest T routed to the streaming path by MOE_PATH_AUTO (env MOE_STREAM_MAX_T overrides).
// Largest T the automatic choice sends down the streaming path. Measured at the
// real shape: the streaming path is ahead at every T it takes (T = 5: 79 vs
// 172 us, T = 40: 262 vs 366 us, T = 64: 297 vs 374 us), so by default it takes
// all of them. MOE_STREAM_MAX_T lowers the limit.
int stream_limit() {
    int lim = MOE_STREAM_MAX_TOKENS;
    if (const char* s = std::getenv("MOE_STREAM_MAX_T")) {
        const int v = std::atoi(s);
        if (v >= 0) lim = v;
    }
    return lim < MOE_STREAM_MAX_TOKENS ? lim : MOE_STREAM_MAX_TOKENS;
}

bool stream_fits(const moe_dims& d) {
    return d.hidden <= 3072 && d.expert_inter <= 1024 && d.dense_inter <= 4096;
}

// Records the stage events of a debug struct around each launch.
struct Stages {
    moe_debug* dbg;
    hipStream_t s;
    int n = 0;
    hipError_t begin(const char* name) {
        if (!dbg) return hipSuccess;
        if (n < MOE_MAX_STAGES) dbg->stage_name[n] = name;
        hipError_t e = hipSuccess;
        if (n <= MOE_MAX_STAGES && dbg->stage_event[n]) e = hipEventRecord(dbg->stage_event[n], s);
        ++n;
        return e;
    }
    hipError_t end() {
        if (!dbg) return hipSuccess;
        dbg->n_stages = n;
        if (n <= MOE_MAX_STAGES && dbg->stage_event[n]) return hipEventRecord(dbg->stage_event[n], s);
        return hipSuccess;
    }
};

template <typename T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

// Device address of `scratch` on the current device, looked up on the first
// call made with that device current and kept for the later ones.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_of_current_device(void** out) {
    int dev = -1;
    HIP_TRY(hipGetDevice(&dev), "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
        if (!p) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) gave a null address on device %d", dev);
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

// moe_ffn_layer's workspace: the block's, then the two branches' bf16 inputs
struct FfnLayout {
    size_t total;
};
FfnLayout ffn_layout(const moe_dims& d, int64_t T) {
    return {make_layout(d, T).total + 2 * up256((size_t)T * d.hidden * 2)};
}

// Checks shared by moe_ffn_layer and moe_prefill_chunked (the workspace size
// is each caller's own). layer: the norm kernels run (n may still be NULL).
int check_layer_args(const moe_dims* d, const moe_weights* w, const moe_ffn_norms* n, bool layer, const void* h,
                     int32_t T, const void* out, const void* ws) {
    int rc;
    if ((rc = check_dims(d)) || (rc = check_T(T)) || (rc = check_weights(w)) || (rc = check_tiled(w))) return rc;
    if (layer && d->hidden > kFfnMaxHidden)
        return fail(MOE_ERR_UNSUPPORTED, "hidden=%d: the feed-forward norms take hidden <= %d", d->hidden,
                    kFfnMaxHidden);
    if (n) {
        const void* gains[] = {n->pre_dense, n->pre_moe, n->post_dense, n->post_moe, n->post};
        const char* names[] = {"pre_dense", "pre_moe", "post_dense", "post_moe", "post"};
        for (int i = 0; i < 5; ++i)
            if (gains[i] && !aligned(gains[i], 16))
                return fail(MOE_ERR_ALIGN, "norm gain %s is not 16-byte aligned", names[i]);
        if (!(n->eps >= 0.f) || n->eps > 1.f) return fail(MOE_ERR_SHAPE, "norm eps=%g must be in [0, 1]", (double)n->eps);
    }
    if (T > 0) {  // empty batch: h, out and ws may be NULL
        CHECK_PTR(h, "h", 16);
        CHECK_PTR(out, "out", 16);
        if (out == h) return fail(MOE_ERR_SHAPE, "out may not alias h");
        if (!ws) return fail(MOE_ERR_NULL, "workspace is NULL");
        if (!aligned(ws, 256)) return fail(MOE_ERR_ALIGN, "workspace must be 256-byte aligned");
    }
    return MOE_OK;
}

// The block's pipeline. The router reads x as given, the experts x or its
// MoE pre-norm, the dense MLP x or its dense pre-norm; without norms y = dense
// + moe (moe_block), with them (moe_ffn_layer) the last stage forms
// y = h + N_post(N_post_dense(dense) + N_post_moe(moe)).
// Arguments are checked by the callers.
int block_impl(const moe_dims* d, const moe_weights* w, const void* x, const void* xd_in, int32_t T, void* y,
               const moe_ffn_norms* norms, const void* hres, moe_debug* dbg, void* ws, hipStream_t stream) {
    // the per-row E4M3 quantisers hold a row in registers
    if (w->expert_dtype == MOE_DTYPE_FP8 && (d->hidden > 16384 || d->expert_inter > 16384))
        return fail(MOE_ERR_UNSUPPORTED, "E4M3 experts take hidden and expert_inter <= 16384");
    int path = dbg ? dbg->path : MOE_PATH_AUTO;
    if (path != MOE_PATH_AUTO && path != MOE_PATH_STREAM && path != MOE_PATH_GROUPED)
        return fail(MOE_ERR_UNSUPPORTED, "unknown path %d", path);
    if (path == MOE_PATH_AUTO)
        path = (T <= stream_limit() && stream_fits(*d)) ? MOE_PATH_STREAM : MOE_PATH_GROUPED;
    if (path == MOE_PATH_STREAM && (T > MOE_STREAM_MAX_TOKENS || !stream_fits(*d)))
        return fail(MOE_ERR_UNSUPPORTED,
                    "streaming path needs T <= %d, hidden <= 3072, expert_inter <= 1024, dense_inter <= 4096",
                    MOE_STREAM_MAX_TOKENS);
    g_err[0] = 0;
    if (dbg) {
        dbg->path_taken = path;
        dbg->n_stages = 0;
    }
    if (T == 0) return MOE_OK;

    const Layout L = make_layout(*d, T);
    // experts' weight format for the kernels: 0 bf16, 1 int8, 2 E4M3
    const int wq = w->expert_dtype == MOE_DTYPE_FP8 ? 2 : w->expert_dtype == MOE_DTYPE_INT8 ? 1 : 0;
    const int H = d->hidden, E = d->num_experts, K = d->top_k, I = d->expert_inter, Id = d->dense_inter;
    int32_t* topk_idx = at<int32_t>(ws, L.topk_idx);
    float* topk_w = at<float>(ws, L.topk_w);
    int32_t* pair_rank = at<int32_t>(ws, L.pair_rank);
    moe::PermuteOut po{};
    po.tile_counts = at<int32_t>(ws, L.tile_counts);
    po.counts = at<int32_t>(ws, L.counts);
    po.offsets = at<int32_t>(ws, L.offsets);
    po.perm_token = at<int32_t>(ws, L.perm_token);
    po.perm_w = at<float>(ws, L.perm_w);
    po.inv_row = at<int32_t>(ws, L.inv_row);
    po.active = at<int32_t>(ws, L.active);
    po.n_active = at<int32_t>(ws, L.n_active);
    po.mtile_group = at<int32_t>(ws, L.mtile_group);
    po.mtile_row0 = at<int32_t>(ws, L.mtile_row0);
    po.n_mtiles = at<int32_t>(ws, L.n_mtiles);
    po.tiles[0] = at<int2>(ws, L.gemm_tiles[0]);
    po.tiles[1] = at<int2>(ws, L.gemm_tiles[1]);
    po.n_nt[0] = moe::gemm_n_tiles_gateup(I);
    po.n_nt[1] = moe::gemm_n_tiles_down(H);
    po.max_mtiles = L.max_mtiles;
    uint16_t* h = at<uint16_t>(ws, L.h);
    uint16_t* hd = at<uint16_t>(ws, L.hd);
    uint16_t* rows = at<uint16_t>(ws, L.rows);
    const uint16_t* xb = (const uint16_t*)x;
    const uint16_t* xdb = (const uint16_t*)xd_in;
    // the router normalises its own input (a scale-free RMSNorm), so it reads
    // the un-normalised stream even where the experts read a pre-norm of it
    const uint16_t* xr = (const uint16_t*)x;
    const uint16_t* g_pd = norms ? (const uint16_t*)norms->post_dense : nullptr;
    const uint16_t* g_pm = norms ? (const uint16_t*)norms->post_moe : nullptr;
    const uint16_t* g_p = norms ? (const uint16_t*)norms->post : nullptr;

    Stages st{dbg, stream};
    const bool pre = norms && (norms->pre_dense || norms->pre_moe);
    uint16_t* xn_d = nullptr;
    uint16_t* xn_m = nullptr;
    const uint16_t* hb = xb;  // the residual stream the pre-norms read
    if (pre) {
        // the branches' normalised inputs, after the block's own workspace
        const size_t xoff = L.total;
        xn_d = norms->pre_dense ? at<uint16_t>(ws, xoff) : nullptr;
        xn_m = norms->pre_moe ? at<uint16_t>(ws, xoff + up256((size_t)T * H * 2)) : nullptr;
        if (path != MOE_PATH_STREAM) {  // the streaming path forms them in its first launch
            HIP_TRY(st.begin("ffn_prenorm"), "event record");
            HIP_TRY(moe::launch_ffn_prenorm(xb, T, H, (const uint16_t*)norms->pre_dense,
                                            (const uint16_t*)norms->pre_moe, norms->eps, xn_d, xn_m, stream),
                    "ffn_prenorm launch");
        }
        if (xn_d) xdb = xn_d;
        if (xn_m) xb = xn_m;
    }
    if (path == MOE_PATH_STREAM) {
        moe::StreamArgs sa{};
        sa.T = T; sa.H = H; sa.I = I; sa.Id = Id; sa.K = K; sa.E = E;
        sa.x = xb; sa.xr = xr; sa.xd = xdb;
        if (pre) {
            sa.pre_src = hb;
            sa.pre_gd = (const uint16_t*)norms->pre_dense;
            sa.pre_gm = (const uint16_t*)norms->pre_moe;
            sa.pre_eps = norms->eps;
            sa.pre_xd = xn_d;
            sa.pre_xm = xn_m;
        }
        sa.gu = w->expert_gate_up; sa.gu_scale = w->gate_up_scale;
        sa.dw = w->expert_down; sa.dw_scale = w->down_scale;
        sa.counts = po.counts; sa.offsets = po.offsets; sa.active = po.active; sa.n_active = po.n_active;
        sa.perm_token = po.perm_token; sa.perm_w = po.perm_w; sa.inv_row = po.inv_row;
        sa.topk_w = topk_w;
        sa.max_active = T * K < E ? T * K : E;
        sa.dgu = (const uint16_t*)w->dense_gate_up; sa.ddw = (const uint16_t*)w->dense_down;
        sa.h = h; sa.hd = hd; sa.y = (uint16_t*)y;
        sa.part = at<float>(ws, L.part); sa.dpart = at<float>(ws, L.dpart);
        sa.dgu_part = at<float>(ws, L.dgu_part);
        sa.hpart = at<float>(ws, L.hpart);
        sa.with_dense = 1;  // the dense MLP's items ride along in K2, K3 and K4
        if (wq == 2) {  // quantised per token by decode_front's last workgroups
            sa.xq = at<uint16_t>(ws, L.xq);
            sa.x_scale = at<float>(ws, L.xscale);
        }
        HIP_TRY(st.begin("decode_front"), "event record");
        float* lpart = at<float>(ws, L.lpart);
        float* ss_part = at<float>(ws, L.ss_part);
        HIP_TRY(moe::launch_decode_front(sa, (const uint16_t*)w->router_scale, (const uint16_t*)w->router_w,
                                         lpart, ss_part, stream),
                "decode_front launch");
        HIP_TRY(st.begin("decode_route"), "event record");
        HIP_TRY(moe::launch_decode_route(sa, lpart, ss_part, w->logit_bias, w->per_expert_scale, d->rms_eps,
                                         topk_idx, topk_w, stream),
                "decode_route launch");
        HIP_TRY(st.begin("decode_experts_gateup"), "event record");
        HIP_TRY(moe::launch_decode_experts_gateup(sa, wq, stream), "decode_experts_gateup launch");
        if (wq == 2) {
            sa.h_scale = at<float>(ws, L.hscale);
            HIP_TRY(st.begin("h_quant"), "event record");
            HIP_TRY(moe::launch_decode_hquant(sa, stream), "decode_hquant launch");
        }
        HIP_TRY(st.begin("decode_down"), "event record");
        HIP_TRY(moe::launch_decode_down(sa, wq, stream), "decode_down launch");
        if (norms) {
            HIP_TRY(st.begin("ffn_post"), "event record");
            HIP_TRY(moe::launch_ffn_post((const uint16_t*)hres, sa.dpart, sa.part, true, po.inv_row, topk_w, T, H,
                                         K, g_pd, g_pm, g_p, norms->eps, (uint16_t*)y, stream),
                    "ffn_post launch");
        } else {
            HIP_TRY(st.begin("decode_combine"), "event record");
            HIP_TRY(moe::launch_decode_combine(sa, stream), "decode_combine launch");
        }
    } else {
        HIP_TRY(st.begin("router"), "event record");
        HIP_TRY(moe::launch_router_mfma(xr, (const uint16_t*)w->router_scale,
                                        (const uint16_t*)w->router_w, w->logit_bias,
                                        w->per_expert_scale, T, H, E, K, d->rms_eps, topk_idx,
                                        topk_w, at<float>(ws, L.partial), stream),
                "router launch");
        HIP_TRY(st.begin("permute"), "event record");
        HIP_TRY(moe::launch_permute(topk_idx, topk_w, pair_rank, T, K, E, moe::kGemmBM, po, stream),
                "permute launch");
        moe::GemmArgs g{};
        // experts gate/up + GELU: gathered rows of x (E4M3 experts: of x
        // quantised per token, with the token scales applied before the GELU)
        g.A = xb; g.lda = H; g.a_rows = po.perm_token;
        if (wq == 2) {  // E4M3 code bytes for the fp8 MFMAs (H is a multiple of 256)
            HIP_TRY(st.begin("act_quant"), "event record");
            HIP_TRY(moe::launch_act_quant_fp8_bytes(xb, T, H, at<uint8_t>(ws, L.xq), H, at<float>(ws, L.xscale),
                                                    nullptr, nullptr, stream),
                    "act_quant launch");
            g.A = at<uint16_t>(ws, L.xq);
            g.lda = H;
            g.a_scale = at<float>(ws, L.xscale);
        }
        g.B = w->expert_gate_up; g.b_group_stride = (int64_t)2 * I * H; g.ldb = H;
        g.b_scale = wq ? w->gate_up_scale : nullptr; g.scale_group_stride = 2 * I;
        g.K = H; g.n_out = I; g.up_off = I;
        g.mtile_group = po.mtile_group; g.mtile_row0 = po.mtile_row0; g.n_mtiles = po.n_mtiles;
        g.group_end = po.offsets; g.max_mtiles = L.max_mtiles; g.tiles = po.tiles[0];
        g.C = h; g.ldc = I;
        // dense gate/up + GELU, in the same launch
        moe::GemmArgs gd{};
        gd.A = xdb; gd.lda = H; gd.B = w->dense_gate_up; gd.ldb = H; gd.K = H;
        gd.n_out = Id; gd.up_off = Id; gd.M_dense = T; gd.C = hd; gd.ldc = Id;
        HIP_TRY(st.begin("gemm_gateup"), "event record");
        HIP_TRY(moe::launch_gemm_gateup(g, &gd, wq, stream), "gemm_gateup launch");
        // experts down, weighted rows
        moe::GemmArgs gw{};
        gw.A = h; gw.lda = I; gw.B = w->expert_down; gw.b_group_stride = (int64_t)H * I; gw.ldb = I;
        gw.b_scale = wq ? w->down_scale : nullptr; gw.scale_group_stride = H;
        gw.K = I; gw.n_out = H;
        gw.mtile_group = po.mtile_group; gw.mtile_row0 = po.mtile_row0; gw.n_mtiles = po.n_mtiles;
        gw.group_end = po.offsets; gw.max_mtiles = L.max_mtiles; gw.tiles = po.tiles[1];
        gw.C = rows; gw.ldc = H; gw.row_w = po.perm_w;
        if (wq == 2) {
            // h quantised per row to code bytes (rows padded with zero codes to
            // whole K-steps); each row's factor becomes router weight x scale
            const int ldh = moe::fp8_row_bytes(I);
            HIP_TRY(st.begin("h_quant"), "event record");
            HIP_TRY(moe::launch_act_quant_fp8_bytes(h, (int64_t)T * K, I, at<uint8_t>(ws, L.hq), ldh,
                                                    at<float>(ws, L.hscale), po.perm_w, at<float>(ws, L.wrow),
                                                    stream),
                    "h_quant launch");
            gw.A = at<uint16_t>(ws, L.hq);
            gw.lda = ldh;
            gw.row_w = at<float>(ws, L.wrow);
        }
        // dense down (fp32), in the same launch
        float* dout = at<float>(ws, L.dout);
        moe::GemmArgs gc{};
        gc.A = hd; gc.lda = Id; gc.B = w->dense_down; gc.ldb = Id; gc.K = Id; gc.n_out = H;
        gc.M_dense = T; gc.Cf = dout; gc.ldc = H;
        HIP_TRY(st.begin("gemm_down"), "event record");
        HIP_TRY(moe::launch_gemm_down(gw, &gc, wq, stream), "gemm_down launch");
        if (norms) {
            HIP_TRY(st.begin("ffn_post"), "event record");
            HIP_TRY(moe::launch_ffn_post((const uint16_t*)hres, dout, rows, false, po.inv_row, nullptr, T, H, K,
                                         g_pd, g_pm, g_p, norms->eps, (uint16_t*)y, stream),
                    "ffn_post launch");
        } else {
            HIP_TRY(st.begin("combine"), "event record");
            HIP_TRY(moe::launch_combine(dout, rows, po.inv_row, T, H, K, (uint16_t*)y, stream),
                    "combine launch");
        }
    }
    HIP_TRY(st.end(), "event record");

    if (dbg) {
        const int64_t TK = (int64_t)T * K;
        struct { void* dst; const void* src; size_t bytes; } cp[] = {
            {dbg->topk_idx, topk_idx, (size_t)TK * 4},
            {dbg->topk_w, topk_w, (size_t)TK * 4},
            {dbg->counts, po.counts, (size_t)E * 4},
            {dbg->offsets, po.offsets, (size_t)(E + 1) * 4},
            {dbg->perm_token, po.perm_token, (size_t)TK * 4},
            {dbg->inv_row, po.inv_row, (size_t)TK * 4},
        };
        for (auto& c : cp)
            if (c.dst) HIP_TRY(hipMemcpyAsync(c.dst, c.src, c.bytes, hipMemcpyDeviceToDevice, stream),
                               "debug copy");
    }
    return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_last_error(void) { return g_err; }

size_t moe_workspace_bytes(const moe_dims* d, int32_t T) {
    if (check_dims(d) != MOE_OK || check_T(T) != MOE_OK) return 0;
    return make_layout(*d, T).total;
}

int moe_route(const moe_dims* d, const moe_weights* w, const void* x, int32_t T, int32_t* topk_idx,
              float* topk_w, void* ws, size_t ws_bytes, hipStream_t stream) {
    int rc;
    if ((rc = check_dims(d)) || (rc = check_T(T)) || (rc = check_weights(w))) return rc;
    g_err[0] = 0;
    if (T == 0) return MOE_OK;  // empty batch: tensors may be NULL, nothing is launched
    CHECK_PTR(x, "x", 16);
    CHECK_PTR(topk_idx, "topk_idx", 4);
    CHECK_PTR(topk_w, "topk_w", 4);
    if ((rc = check_ws(d, T, ws, ws_bytes))) return rc;
    const Layout L = make_layout(*d, T);
    if (T > kRouterMfmaMinT || d->hidden > kRouterLogitsMaxHidden) {
        HIP_TRY(moe::launch_router_mfma((const uint16_t*)x, (const uint16_t*)w->router_scale,
                                        (const uint16_t*)w->router_w, w->logit_bias,
                                        w->per_expert_scale, T, d->hidden, d->num_experts, d->top_k,
                                        d->rms_eps, topk_idx, topk_w, at<float>(ws, L.partial), stream),
                "router launch");
        return MOE_OK;
    }
    float* logits = at<float>(ws, L.logits);
    HIP_TRY(moe::launch_router_logits((const uint16_t*)x, (const uint16_t*)w->router_scale,
                                      (const uint16_t*)w->router_w, w->logit_bias, T, d->hidden,
                                      d->num_experts, d->rms_eps, logits, stream),
            "router_logits launch");
    HIP_TRY(moe::launch_router_topk(logits, w->per_expert_scale, T, d->num_experts, d->top_k,
                                    topk_idx, topk_w, stream),
            "router_topk launch");
    return MOE_OK;
}

int moe_block(const moe_dims* d, const moe_weights* w, const void* x, int32_t T, void* y,
              moe_debug* dbg, void* ws, size_t ws_bytes, hipStream_t stream) {
    int rc;
    if ((rc = check_dims(d)) || (rc = check_T(T)) || (rc = check_weights(w)) || (rc = check_tiled(w))) return rc;
    if (T > 0) {  // empty batch: x, y and ws may be NULL
        CHECK_PTR(x, "x", 16);
        CHECK_PTR(y, "y", 16);
        if ((rc = check_ws(d, T, ws, ws_bytes))) return rc;
    }
    return block_impl(d, w, x, x, T, y, nullptr, nullptr, dbg, ws, stream);
}

int moe_block_noalloc(const moe_dims* d, const moe_weights* w, const void* x, int32_t T, void* y,
                      moe_debug* dbg, hipStream_t stream) {
    int rc;
    if ((rc = check_dims(d)) || (rc = check_T(T)) || (rc = check_weights(w)) || (rc = check_tiled(w))) return rc;
    if (T == 0) return block_impl(d, w, x, x, T, y, nullptr, nullptr, dbg, nullptr, stream);
    CHECK_PTR(x, "x", 16);
    CHECK_PTR(y, "y", 16);
    const size_t need = make_layout(*d, T).total;
    if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
        return fail(MOE_ERR_WORKSPACE,
                    "moe_block_noalloc: T=%d needs %zu bytes of scratch, more than the %zu the library holds "
                    "(moe_block with a workspace takes any size)", T, need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    if ((rc = scratch_of_current_device(&ws))) return rc;
    return block_impl(d, w, x, x, T, y, nullptr, nullptr, dbg, ws, stream);
}

size_t moe_ffn_workspace_bytes(const moe_dims* d, int32_t T) {
    if (check_dims(d) != MOE_OK || check_T(T) != MOE_OK) return 0;
    return ffn_layout(*d, T).total;
}

int moe_ffn_layer(const moe_dims* d, const moe_weights* w, const moe_ffn_norms* n, const void* h, int32_t T,
                  void* out, moe_debug* dbg, void* ws, size_t ws_bytes, hipStream_t stream) {
    int rc;
    if ((rc = check_layer_args(d, w, n, true, h, T, out, ws))) return rc;
    moe_ffn_norms none{};
    if (!n) n = &none;
    if (T > 0) {
        const size_t need = ffn_layout(*d, T).total;
        if (ws_bytes < need)
            return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes < %zu needed at T=%d", ws_bytes, need, T);
    }
    return block_impl(d, w, h, h, T, out, n, h, dbg, ws, stream);
}

int32_t moe_prefill_chunk_tokens(int32_t chunk_tokens) {
    if (chunk_tokens <= 0) return kPrefillChunkDefault;
    const int32_t c = chunk_tokens / kSlidingWindow * kSlidingWindow;
    return c < kSlidingWindow ? kSlidingWindow : (c > kPrefillChunkMax ? kPrefillChunkMax : c);
}

size_t moe_prefill_workspace_bytes(const moe_dims* d, int32_t chunk_tokens) {
    if (check_dims(d) != MOE_OK) return 0;
    return ffn_layout(*d, moe_prefill_chunk_tokens(chunk_tokens)).total;
}

int moe_prefill_chunked(const moe_dims* d, const moe_weights* w, const moe_ffn_norms* n, const void* h,
                        int32_t T, int32_t chunk_tokens, void* out, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
    int rc;
    if ((rc = check_layer_args(d, w, n, n != nullptr, h, T, out, ws))) return rc;
    const int32_t C = moe_prefill_chunk_tokens(chunk_tokens);
    if (T > 0) {  // the chunks have two sizes at most: the first's and the ragged last one's
        auto need_at = [&](int32_t t) { return n ? ffn_layout(*d, t).total : make_layout(*d, t).total; };
        const int32_t first = T < C ? T : C, last = T - (T - 1) / C * C;
        const size_t need = std::max(need_at(first), need_at(last));
        if (ws_bytes < need)
            return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes < %zu needed for chunks of %d tokens", ws_bytes,
                        need, first);
    }
    g_err[0] = 0;
    const size_t row = (size_t)d->hidden * 2;
    for (int32_t t0 = 0; t0 < T; t0 += C) {
        const int32_t tc = T - t0 < C ? T - t0 : C;
        const void* hc = static_cast<const char*>(h) + (size_t)t0 * row;
        void* oc = static_cast<char*>(out) + (size_t)t0 * row;
        if ((rc = block_impl(d, w, hc, hc, tc, oc, n, n ? hc : nullptr, nullptr, ws, stream))) return rc;
    }
    return MOE_OK;
}

int dense_mlp(const moe_dims* d, const void* dense_gate_up, const void* dense_down, const void* x,
              int32_t T, void* y, void* ws, size_t ws_bytes, hipStream_t stream) {
    int rc;
    if ((rc = check_dims(d)) || (rc = check_T(T))) return rc;
    CHECK_PTR(dense_gate_up, "dense_gate_up", 16);
    CHECK_PTR(dense_down, "dense_down", 16);
    g_err[0] = 0;
    if (T == 0) return MOE_OK;  // empty batch: x, y and ws may be NULL
    CHECK_PTR(x, "x", 16);
    CHECK_PTR(y, "y", 16);
    if ((rc = check_ws(d, T, ws, ws_bytes))) return rc;
    const Layout L = make_layout(*d, T);
    const int H = d->hidden, Id = d->dense_inter;
    uint16_t* hd = at<uint16_t>(ws, L.hd);
    if (T <= stream_limit() && stream_fits(*d)) {
        moe::StreamArgs sa{};
        sa.T = T; sa.H = H; sa.I = d->expert_inter; sa.Id = Id; sa.K = d->top_k; sa.E = d->num_experts;
        sa.x = (const uint16_t*)x; sa.xr = sa.x; sa.xd = sa.x; sa.max_active = 0; sa.with_dense = 1; sa.front_dense = 1;
        sa.dgu = (const uint16_t*)dense_gate_up; sa.ddw = (const uint16_t*)dense_down;
        sa.hd = hd; sa.y = (uint16_t*)y;
        sa.part = at<float>(ws, L.part); sa.dpart = at<float>(ws, L.dpart);
        sa.dgu_part = at<float>(ws, L.dgu_part);
        HIP_TRY(moe::launch_decode_front(sa, nullptr, nullptr, nullptr, nullptr, stream),
                "decode_front launch");
        HIP_TRY(moe::launch_decode_experts_gateup(sa, 0, stream), "dense finish launch");
        HIP_TRY(moe::launch_decode_down(sa, 0, stream), "decode_down launch");
        HIP_TRY(moe::launch_decode_combine(sa, stream), "decode_combine launch");
    } else {
        moe::GemmArgs gd{};
        gd.A = (const uint16_t*)x; gd.lda = H; gd.B = dense_gate_up; gd.ldb = H; gd.K = H;
        gd.n_out = Id; gd.up_off = Id; gd.M_dense = T; gd.C = hd; gd.ldc = Id;
        HIP_TRY(moe::launch_gemm_gateup(gd, nullptr, 0, stream), "gemm_gateup dense launch");
        moe::GemmArgs gc{};
        gc.A = hd; gc.lda = Id; gc.B = dense_down; gc.ldb = Id; gc.K = Id; gc.n_out = H;
        gc.M_dense = T; gc.C = (uint16_t*)y; gc.ldc = H;
        HIP_TRY(moe::launch_gemm_down(gc, nullptr, 0, stream), "gemm_down dense launch");
    }
    return MOE_OK;
}

int moe_quantize_int8(const void* w_bf16, int64_t rows, int32_t cols, int8_t* q, float* scale,
                      hipStream_t stream) {
    if (rows < 0 || rows > ((int64_t)1 << 32) || cols <= 0 || cols % 8)
        return fail(MOE_ERR_SHAPE, "rows=%lld cols=%d (need rows >= 0, cols > 0, cols %% 8 == 0)",
                    (long long)rows, cols);
    CHECK_PTR(w_bf16, "w", 16);
    CHECK_PTR(q, "q", 16);
    CHECK_PTR(scale, "scale", 4);
    g_err[0] = 0;
    if (rows == 0) return MOE_OK;
    HIP_TRY(moe::launch_quantize_int8((const uint16_t*)w_bf16, rows, cols, q, scale, stream),
            "quantize launch");
    return MOE_OK;
}

int moe_quantize_fp8(const void* w_bf16, int64_t rows, int32_t cols, uint8_t* q, float* scale,
                     hipStream_t stream) {
    if (rows < 0 || rows > ((int64_t)1 << 32) || cols <= 0 || cols % 8)
        return fail(MOE_ERR_SHAPE, "rows=%lld cols=%d (need rows >= 0, cols > 0, cols %% 8 == 0)",
                    (long long)rows, cols);
    CHECK_PTR(w_bf16, "w", 16);
    CHECK_PTR(q, "q", 16);
    CHECK_PTR(scale, "scale", 4);
    g_err[0] = 0;
    if (rows == 0) return MOE_OK;
    HIP_TRY(moe::launch_quantize_fp8((const uint16_t*)w_bf16, rows, cols, q, scale, stream), "quantize launch");
    return MOE_OK;
}

int moe_tile_weights(const void* src, int64_t rows, int32_t cols, int32_t dtype, void* dst,
                     hipStream_t stream) {
    if (dtype != MOE_DTYPE_BF16 && dtype != MOE_DTYPE_INT8 && dtype != MOE_DTYPE_FP8)
        return fail(MOE_ERR_UNSUPPORTED, "dtype %d", dtype);
    if (rows < 0 || rows % 16 || cols <= 0 || cols % 64)
        return fail(MOE_ERR_SHAPE, "rows=%lld cols=%d (need rows %% 16 == 0, cols %% 64 == 0)",
                    (long long)rows, cols);
    CHECK_PTR(src, "src", 16);
    CHECK_PTR(dst, "dst", 16);
    if (src == dst) return fail(MOE_ERR_SHAPE, "src and dst must be different buffers");
    g_err[0] = 0;
    if (rows == 0) return MOE_OK;
    HIP_TRY(moe::launch_tile_weights(src, rows, cols, dtype != MOE_DTYPE_BF16, dst, stream),
            "tile launch");
    return MOE_OK;
}

}  // extern "C"
