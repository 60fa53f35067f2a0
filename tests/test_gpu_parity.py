"""GPU parity of the HIP path against the CPU oracle (through the C ABI).

Integer results (top-k indices, counts, offsets, grouped order, inverse rows,
int8 codes) must match bit for bit; near-ties of the router (logit gap under
1e-6) are flagged and then checked for validity instead. The block output must
reach cosine >= 0.9999 and relative L2 <= 1e-2 (bf16) or 2e-2 (int8 and E4M3
experts), pooled over the tokens compared and for each token on its own.
Real-shape workloads are checked at their full sizes, in the configuration
the bench times: every token up to T = 2048; at T = 4096 and 16384 the tokens
of the first and last grouped row of every 128 rows of each expert (so every
GEMM M-tile has checked rows) plus a random sample.
"""
import sys

import numpy as np
import pytest
import torch

import moe_synth
import oracle
from mixture_experts_ffn_amd import (MOE_PATH_AUTO, MOE_PATH_GROUPED, MOE_PATH_STREAM, BlockCall, FfnNorms,
                                     MoEError, dense_mlp, moe_block, moe_ffn_layer, moe_prefill_chunk_tokens,
                                     moe_prefill_chunked, moe_prefill_workspace_bytes, moe_quantize_fp8,
                                     moe_quantize_int8,
                                     moe_route, moe_tile_weights, moe_workspace_bytes, new_debug)
from gpu_util import (REL_BF16, REL_INT8, bf16_dev, check_routing, compare_y, dims_of,
                      oracle_int8_weights, oracle_weights, routing_for, to_np, upload, y_f64)

pytestmark = pytest.mark.gpu

_CACHE = {}
_WCACHE = {}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda:0")


def inputs(name, dev, tokens=None):
    """(workload, oracle weights, x, device weights, device x). Workloads that
    draw the same weights (same shape, seed and variant) share one upload."""
    key = (name, tokens)
    if key not in _CACHE:
        wl = moe_synth.WORKLOADS[name]
        wkey = (wl.shape, wl.seed, wl.skew, wl.int8, wl.fp8)
        if wkey not in _WCACHE:
            w = moe_synth.make_weights(wl.shape, wl.seed, wl.skew)
            _WCACHE[wkey] = (w, upload(w, dev, int8=wl.int8, fp8=wl.fp8))
        w, lw = _WCACHE[wkey]
        x = moe_synth.make_tokens(wl.shape, wl.seed, wl.tokens if tokens is None else tokens)
        _CACHE[key] = (wl, w, x, lw, bf16_dev(x, dev))
    return _CACHE[key]


def oracle_route(wl, w, x):
    s = wl.shape
    return oracle.route(x, w["router_scale"], w["router_w"], w["per_expert_scale"], s.top_k,
                        s.rms_eps, w.get("logit_bias"))


def sample_tokens(T, n=24, seed=0):
    if T <= 64:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    s = set(rng.choice(T, size=n - 2, replace=False).tolist()) | {0, T - 1}
    return np.array(sorted(s))


#: every token is compared with the oracle up to this batch size
FULL_CHECK_T = 2048
#: above it, the first and last grouped row of every run of this many rows of
#: each expert (a multiple of the GEMM's 256-row M-tiles and of their halves)
SEGMENT_ROWS = 128


def block_check_tokens(T, dbg, n_random=24, seed=0):
    """Tokens whose y the block tests compare: all of them up to FULL_CHECK_T;
    beyond, the tokens of the first and last grouped row of every SEGMENT_ROWS
    rows of each expert (through the GPU's own offsets and perm_token, so that
    every M-tile of every expert GEMM block, partial last tiles included, has
    rows checked) plus a random sample."""
    if T <= FULL_CHECK_T:
        return np.arange(T)
    off, perm = dbg["offsets"], dbg["perm_token"]
    rows = set()
    for e in range(len(off) - 1):
        for r0 in range(int(off[e]), int(off[e + 1]), SEGMENT_ROWS):
            rows.add(r0)
            rows.add(min(r0 + SEGMENT_ROWS, int(off[e + 1])) - 1)
    toks = {int(perm[r]) for r in rows} | set(sample_tokens(T, n_random, seed).tolist())
    return np.array(sorted(toks))


def compare_per_token(y_gpu, y_ref, rel_max):
    """Beside the pooled cosine and rel-L2: every token's own rel-L2 within the
    same bar. Returns the largest."""
    a = y_gpu.astype(np.float64)
    b = y_ref.astype(np.float64)
    rel = np.linalg.norm(a - b, axis=1) / np.linalg.norm(b, axis=1)
    worst = int(np.argmax(rel))
    assert rel[worst] <= rel_max, f"token row {worst}: rel-L2 {rel[worst]:.3g} > {rel_max}"
    return float(rel[worst])


def run_block(wl, lw, xd, path):
    s = wl.shape
    T = xd.shape[0]
    K, E = s.top_k, s.num_experts
    out = dict(topk_idx=torch.empty((T, K), dtype=torch.int32, device=xd.device),
               topk_w=torch.empty((T, K), dtype=torch.float32, device=xd.device),
               counts=torch.empty(E, dtype=torch.int32, device=xd.device),
               offsets=torch.empty(E + 1, dtype=torch.int32, device=xd.device),
               perm_token=torch.empty(T * K, dtype=torch.int32, device=xd.device),
               inv_row=torch.empty(T * K, dtype=torch.int32, device=xd.device))
    dbg = new_debug(path, **out)
    y = moe_block(dims_of(s), lw, xd, debug=dbg)
    torch.cuda.synchronize()
    assert dbg.path_taken == path
    return y, {k: to_np(v) for k, v in out.items()}


# ----------------------------------------------------------------------------
def _tiled_reference(w: np.ndarray) -> np.ndarray:
    """The tiled layout as the header defines it, from index arithmetic:
    element (r, c) of tile (r // 16, c // 64) sits at lane 16 ((c % 64) // 16)
    + r % 16, position c % 16 of that lane; bf16 tiles store positions 0..7 of
    all lanes, then 8..15; int8 tiles store each lane's 16 positions together."""
    rows, cols = w.shape
    out = np.empty(w.size, dtype=w.dtype)
    tb = 1024 if w.dtype.itemsize == 1 else 2048
    esz = w.dtype.itemsize
    for r in range(rows):
        for c in range(cols):
            tile = (r // 16) * (cols // 64) + c // 64
            lane = 16 * ((c % 64) // 16) + r % 16
            pos = c % 16
            if esz == 1:
                byte = lane * 16 + pos
            else:
                byte = (pos // 8) * 1024 + lane * 16 + (pos % 8) * 2
            out[(tile * tb + byte) // esz] = w[r, c]
    return out


def _tiled(w: np.ndarray) -> np.ndarray:
    """Vectorised form of _tiled_reference (checked against it below)."""
    rows, cols = w.shape
    if w.dtype.itemsize == 1:  # int8 or E4M3 codes: (ti, r, tj, g, pos) -> (ti, tj, g, r, pos)
        return w.reshape(rows // 16, 16, cols // 64, 4, 16).transpose(0, 2, 3, 1, 4).ravel()
    # (ti, r, tj, g, h, e) -> (ti, tj, h, g, r, e)
    return w.reshape(rows // 16, 16, cols // 64, 4, 2, 8).transpose(0, 2, 4, 3, 1, 5).ravel()


@pytest.mark.parametrize("dtype,shape", [("bf16", (48, 192)), ("int8", (32, 128)), ("bf16", (2, 16, 64))])
def test_tile_weights_layout(dev, dtype, shape):
    say(f"case: moe_tile_weights {dtype} {shape}")
    rng = np.random.default_rng(7)
    if dtype == "bf16":
        w = rng.integers(-32768, 32767, size=shape, dtype=np.int16)
        t = moe_tile_weights(torch.from_numpy(w).view(torch.bfloat16).to(dev))
        got = to_np(t.view(torch.int16)).ravel()
    else:
        w = rng.integers(-127, 128, size=shape, dtype=np.int8)
        t = moe_tile_weights(torch.from_numpy(w).to(dev))
        got = to_np(t).ravel()
    torch.cuda.synchronize()
    ref = _tiled_reference(w.reshape(-1, shape[-1]))
    np.testing.assert_array_equal(got, ref)
    np.testing.assert_array_equal(_tiled(w.reshape(-1, shape[-1])), ref)


def test_quantize_fp8_bit_exact(dev):
    """The E4M3 quantiser: codes and scales bit for bit against the oracle's,
    on real-shape expert weights and on rows built to hit ties, subnormal codes
    and zero rows."""
    say("case: fp8 quantiser, real-shape expert weights (seed 5)")
    wl, w, x, lw, xd = inputs("fp8_decode", dev)
    q_ref, s_ref = oracle.quantize_fp8(w["expert_gate_up"][:16])
    q, s = moe_quantize_fp8(bf16_dev(w["expert_gate_up"][:16], dev))
    np.testing.assert_array_equal(to_np(q), q_ref)
    np.testing.assert_array_equal(to_np(s).view(np.uint32), s_ref.view(np.uint32))
    # the full layer as uploaded for the block (quantised, then tiled)
    qd_ref, sd_ref = oracle.quantize_fp8(w["expert_down"])
    np.testing.assert_array_equal(to_np(lw.expert_down).ravel(), _tiled(qd_ref.reshape(-1, qd_ref.shape[-1])))
    np.testing.assert_array_equal(to_np(lw.down_scale).view(np.uint32), sd_ref.view(np.uint32))
    # rows whose scale is a power of two (max 448 * 2^k): every value is exact
    # in fp32 after the division, so halfway cases stay halfway
    rng = np.random.default_rng(9)
    grid = np.array([0.0, 2.0 ** -10, 1.5 * 2.0 ** -9, 2.0 ** -7, 1.0625, 1.1875, 3.25, 100.0, 300.0],
                    dtype=np.float32)
    rows = np.stack([np.concatenate([[448.0], rng.choice(grid, 63) * rng.choice([-1, 1], 63)]) * 2.0 ** k
                     for k in range(-8, 8)] + [np.zeros(64)]).astype(np.float32)
    bits = moe_synth.f32_to_bf16_bits(rows)
    q2_ref, s2_ref = oracle.quantize_fp8(bits)
    q2, s2 = moe_quantize_fp8(bf16_dev(bits, dev))
    np.testing.assert_array_equal(to_np(q2), q2_ref)
    np.testing.assert_array_equal(to_np(s2).view(np.uint32), s2_ref.view(np.uint32))


def test_quantize_int8_bit_exact(dev):
    say("case: int8 quantiser, real-shape expert weights (seed 4)")
    wl, w, x, lw, xd = inputs("int8_decode", dev)
    q_ref, s_ref = oracle.quantize_int8(w["expert_gate_up"][:16])
    gu = bf16_dev(w["expert_gate_up"][:16], dev)
    q, s = moe_quantize_int8(gu)
    np.testing.assert_array_equal(to_np(q), q_ref)
    np.testing.assert_array_equal(to_np(s).view(np.uint32), s_ref.view(np.uint32))
    # the full layer as uploaded for the block (quantised, then tiled)
    qd_ref, sd_ref = oracle.quantize_int8(w["expert_down"])
    np.testing.assert_array_equal(to_np(lw.expert_down).ravel(), _tiled(qd_ref.reshape(-1, qd_ref.shape[-1])))
    np.testing.assert_array_equal(to_np(lw.down_scale).view(np.uint32), sd_ref.view(np.uint32))
    # zero rows and halfway cases
    row = np.array([[127.0, 2.5, 3.5, -2.5, -0.5, 0.49, 126.5, -127.0]], dtype=np.float32)
    rb = moe_synth.f32_to_bf16_bits(np.concatenate([row, np.zeros_like(row)]))
    q2, s2 = moe_quantize_int8(bf16_dev(rb, dev))
    np.testing.assert_array_equal(to_np(q2)[0], [127, 2, 4, -2, 0, 0, 126, -127])
    assert to_np(s2)[1] == 0 and (to_np(q2)[1] == 0).all()


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "skew", "int8_prefill"])
def test_route_parity(dev, name):
    wl, w, x, lw, xd = inputs(name, dev)
    say(f"case: moe_route {name} T={x.shape[0]}")
    idx, wt = moe_route(dims_of(wl.shape), lw, xd)
    torch.cuda.synchronize()
    ref = oracle_route(wl, w, x)
    n_flag = check_routing(to_np(idx), to_np(wt), ref, w["per_expert_scale"])
    say(f"  flagged near-ties: {n_flag} of {x.shape[0]}")


def test_route_parity_wide_rows(dev):
    """moe_route on a small batch of rows wider than the small-batch router
    stages in LDS: it takes the MFMA router instead of failing at launch."""
    s = moe_synth.BlockShape(hidden=12288, num_experts=64, top_k=8, expert_inter=64, dense_inter=64)
    wl = moe_synth.Workload("wide", s, 8, 31)
    w = moe_synth.make_weights(s, 31)
    x = moe_synth.make_tokens(s, 31, 8)
    say("case: moe_route hidden=12288 T=8")
    lw = upload(w, dev)
    idx, wt = moe_route(dims_of(s), lw, bf16_dev(x, dev))
    torch.cuda.synchronize()
    check_routing(to_np(idx), to_np(wt), oracle_route(wl, w, x), w["per_expert_scale"])


PATH_CASES = [("tiny", MOE_PATH_STREAM), ("tiny", MOE_PATH_GROUPED),
              ("decode", MOE_PATH_STREAM), ("decode", MOE_PATH_GROUPED),
              ("prefill", MOE_PATH_GROUPED), ("skew", MOE_PATH_GROUPED),
              ("int8_decode", MOE_PATH_STREAM), ("int8_decode", MOE_PATH_GROUPED),
              ("int8_prefill", MOE_PATH_GROUPED),
              ("mtp_decode", MOE_PATH_STREAM), ("mtp_decode", MOE_PATH_GROUPED),
              ("fp8_decode", MOE_PATH_STREAM), ("fp8_decode", MOE_PATH_GROUPED), ("fp8_prefill", MOE_PATH_GROUPED)]


@pytest.mark.parametrize("name,path", PATH_CASES)
def test_block_parity(dev, name, path):
    wl, w, x, lw, xd = inputs(name, dev)
    s = wl.shape
    T = x.shape[0]
    say(f"case: moe_block {name} T={T} path={path}")
    y, dbg = run_block(wl, lw, xd, path)
    ref = oracle_route(wl, w, x)
    check_routing(dbg["topk_idx"], dbg["topk_w"], ref, w["per_expert_scale"])
    # grouping: exact integer work on the GPU's own indices
    p = oracle.permute_pairs(dbg["topk_idx"], s.num_experts)
    for k in ("counts", "offsets", "perm_token", "inv_row"):
        np.testing.assert_array_equal(dbg[k], p[k], err_msg=k)
    # block output: every token up to T = 2048, beyond that rows of every M-tile
    toks = block_check_tokens(T, dbg)
    r = routing_for(dbg["topk_idx"][toks], {k: v[toks] for k, v in ref.items()}, w["per_expert_scale"])
    ow, fmt = oracle_weights(wl, w)
    y_ref, _ = oracle.moe_block(x[toks], ow, s.top_k, s.rms_eps, expert_dtype=fmt, routing=r)
    bar = REL_BF16 if fmt == "bf16" else REL_INT8
    cos, rel = compare_y(y_f64(y)[toks], y_ref, bar)
    worst = compare_per_token(y_f64(y)[toks], y_ref, bar)
    say(f"  tokens checked {len(toks)}  cos {cos:.7f}  rel-L2 {rel:.3e}  worst token rel-L2 {worst:.3e}")


def test_skew_routing_collapses_to_few_experts(dev):
    wl, w, x, lw, xd = inputs("skew", dev)
    say("case: skew load imbalance")
    y, dbg = run_block(wl, lw, xd, MOE_PATH_GROUPED)
    counts = dbg["counts"]
    assert counts.sum() == x.shape[0] * wl.shape.top_k
    say(f"  experts with rows: {(counts > 0).sum()}, max rows {counts.max()}")
    assert counts.max() > 8 * x.shape[0] * wl.shape.top_k / wl.shape.num_experts


@pytest.mark.parametrize("name", ["tiny", "decode", "int8_decode", "fp8_decode"])
def test_stream_and_grouped_paths_agree(dev, name):
    wl, w, x, lw, xd = inputs(name, dev)
    say(f"case: paths agree {name}")
    y1, d1 = run_block(wl, lw, xd, MOE_PATH_STREAM)
    y2, d2 = run_block(wl, lw, xd, MOE_PATH_GROUPED)
    np.testing.assert_array_equal(d1["topk_idx"], d2["topk_idx"])
    np.testing.assert_array_equal(d1["perm_token"], d2["perm_token"])
    a, b = y_f64(y1), y_f64(y2)
    rel = np.linalg.norm(a - b) / np.linalg.norm(b)
    assert rel < 5e-3, rel


@pytest.mark.parametrize("name,path", [("prefill", MOE_PATH_GROUPED), ("decode", MOE_PATH_STREAM)])
def test_block_is_deterministic(dev, name, path):
    wl, w, x, lw, xd = inputs(name, dev)
    say(f"case: determinism {name} path={path}")
    y1, _ = run_block(wl, lw, xd, path)
    y2, _ = run_block(wl, lw, xd, path)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_tokens_are_independent(dev):
    wl, w, x, lw, xd = inputs("prefill", dev)
    say("case: batch vs decode slices")
    y_all, _ = run_block(wl, lw, xd, MOE_PATH_GROUPED)
    for t0 in (0, 1000, 2040):
        y8, _ = run_block(wl, lw, xd[t0:t0 + 8].contiguous(), MOE_PATH_STREAM)
        a, b = y_f64(y8), y_f64(y_all[t0:t0 + 8])
        assert np.linalg.norm(a - b) / np.linalg.norm(b) < 5e-3


@pytest.mark.parametrize("name,T", [("tiny", 64), ("decode", 8), ("prefill", 300)])
def test_dense_mlp_parity(dev, name, T):
    wl, w, x, lw, xd = inputs(name, dev)
    say(f"case: dense_mlp {name} T={T}")
    xs = xd[:T].contiguous()
    y = dense_mlp(dims_of(wl.shape), lw.dense_gate_up, lw.dense_down, xs)
    torch.cuda.synchronize()
    y_ref = oracle.dense_mlp(x[:T], w["dense_gate_up"], w["dense_down"])
    compare_y(y_f64(y), y_ref, REL_BF16)
    compare_per_token(y_f64(y), y_ref, REL_BF16)


EDGE = {
    "e1k1": moe_synth.BlockShape(hidden=256, num_experts=1, top_k=1, expert_inter=64, dense_inter=64),
    "k_eq_e": moe_synth.BlockShape(hidden=512, num_experts=8, top_k=8, expert_inter=128, dense_inter=128),
    "e256": moe_synth.BlockShape(hidden=256, num_experts=256, top_k=8, expert_inter=64, dense_inter=192),
}


@pytest.mark.parametrize("shape", sorted(EDGE))
@pytest.mark.parametrize("T,path", [(1, MOE_PATH_STREAM), (1, MOE_PATH_GROUPED), (64, MOE_PATH_STREAM),
                                    (200, MOE_PATH_GROUPED)])
def test_edge_shapes(dev, shape, T, path):
    s = EDGE[shape]
    say(f"case: edge {shape} T={T} path={path}")
    wl = moe_synth.Workload(shape, s, T, 21)
    w = moe_synth.make_weights(s, 21)
    x = moe_synth.make_tokens(s, 21, T)
    lw = upload(w, dev)
    y, dbg = run_block(wl, lw, bf16_dev(x, dev), path)
    ref = oracle_route(wl, w, x)
    check_routing(dbg["topk_idx"], dbg["topk_w"], ref, w["per_expert_scale"])
    p = oracle.permute_pairs(dbg["topk_idx"], s.num_experts)
    for k in ("counts", "offsets", "perm_token", "inv_row"):
        np.testing.assert_array_equal(dbg[k], p[k], err_msg=k)
    r = routing_for(dbg["topk_idx"], ref, w["per_expert_scale"])
    y_ref, _ = oracle.moe_block(x, w, s.top_k, s.rms_eps, routing=r)
    compare_y(y_f64(y), y_ref, REL_BF16)


@pytest.mark.parametrize("T", [65, 129, 1000])
def test_ragged_real_shape(dev, T):
    wl, w, x, lw, xd = inputs("prefill", dev)
    say(f"case: ragged real shape T={T}")
    xs = xd[:T].contiguous()
    y, dbg = run_block(wl, lw, xs, MOE_PATH_GROUPED)
    ref = oracle_route(wl, w, x[:T])
    check_routing(dbg["topk_idx"], dbg["topk_w"], ref, w["per_expert_scale"])
    toks = block_check_tokens(T, dbg)
    r = routing_for(dbg["topk_idx"][toks], {k: v[toks] for k, v in ref.items()}, w["per_expert_scale"])
    y_ref, _ = oracle.moe_block(x[:T][toks], w, 8, 1e-6, routing=r)
    compare_y(y_f64(y)[toks], y_ref, REL_BF16)
    compare_per_token(y_f64(y)[toks], y_ref, REL_BF16)


def test_empty_batch_and_errors(dev):
    wl, w, x, lw, xd = inputs("tiny", dev)
    say("case: empty batch, workspace and path errors")
    d = dims_of(wl.shape)
    y = moe_block(d, lw, xd[:0].contiguous())
    assert y.shape == (0, wl.shape.hidden)
    small = torch.empty(256, dtype=torch.uint8, device=dev)
    with pytest.raises(MoEError, match="WORKSPACE"):
        moe_block(d, lw, xd, workspace=small)
    with pytest.raises(MoEError, match="UNSUPPORTED"):
        wl2, w2, x2, lw2, xd2 = inputs("prefill", dev)
        moe_block(dims_of(wl2.shape), lw2, xd2[:100].contiguous(), debug=new_debug(MOE_PATH_STREAM))


@pytest.mark.parametrize("name,path", [("tiny", MOE_PATH_STREAM), ("tiny", MOE_PATH_GROUPED),
                                       ("decode", MOE_PATH_STREAM), ("fp8_decode", MOE_PATH_STREAM),
                                       ("fp8_decode", MOE_PATH_GROUPED)])
def test_graph_replay(dev, name, path):
    """The block captured into a HIP graph: every replay, with eager calls of
    the block on other tokens (same workspace) and synchronisations between
    the replays, gives the eager result bit for bit (no kernel depends on
    scratch left by an earlier call, and the kernels are deterministic)."""
    wl, w, x, lw, xd = inputs(name, dev)
    say(f"case: graph replay {name} path={path}")
    d = dims_of(wl.shape)
    T = xd.shape[0]
    ws = torch.empty(moe_workspace_bytes(d, T), dtype=torch.uint8, device=dev)
    y_eager = moe_block(d, lw, xd, debug=new_debug(path), workspace=ws).clone()
    torch.cuda.synchronize()
    y_g = torch.empty_like(y_eager)
    call = BlockCall(d, lw, xd, y=y_g, workspace=ws)
    dbg = new_debug(path)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(dbg)
    torch.cuda.synchronize()
    x_other = torch.flip(xd, dims=[0]).contiguous()
    for rep in range(3):
        y_g.zero_()
        moe_block(d, lw, x_other, debug=new_debug(path), workspace=ws)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_g, y_eager), f"replay {rep} differs from the eager result"


# ---------------------------------------------------------------- the layer's FFN around the block
FFN_SETS = {"all": oracle.FFN_NORMS, "post_only": ("post",), "pre_moe": ("pre_moe", "post_moe"),
            "pre_dense": ("pre_dense", "post_dense"), "none": ()}


def ffn_gains(H, which, dev, eps=1e-5):
    """Seeded bf16 gains 1 + 0.1 N for the norms in FFN_SETS[which] (the rest
    absent): (the oracle's dict, the library's FfnNorms)."""
    rng = np.random.default_rng(7)
    gains = {k: moe_synth.f32_to_bf16_bits((1.0 + 0.1 * rng.standard_normal(H)).astype(np.float32))
             for k in oracle.FFN_NORMS}
    sel = FFN_SETS[which]
    norms_np = {**{k: (gains[k] if k in sel else None) for k in oracle.FFN_NORMS}, "eps": eps}
    norms = FfnNorms(**{k: (torch.from_numpy(gains[k].view(np.int16)).view(torch.bfloat16).to(dev)
                            if k in sel else None) for k in oracle.FFN_NORMS}, eps=eps)
    return norms_np, norms


@pytest.mark.parametrize("name,path,which", [
    ("tiny", MOE_PATH_STREAM, "all"), ("tiny", MOE_PATH_GROUPED, "all"), ("tiny", MOE_PATH_GROUPED, "none"),
    ("decode", MOE_PATH_STREAM, "all"), ("decode", MOE_PATH_STREAM, "post_only"),
    ("decode", MOE_PATH_GROUPED, "pre_moe"), ("prefill", MOE_PATH_GROUPED, "all"),
    ("int8_decode", MOE_PATH_STREAM, "all"), ("fp8_decode", MOE_PATH_STREAM, "all"),
    ("fp8_decode", MOE_PATH_GROUPED, "pre_moe"), ("decode", MOE_PATH_STREAM, "pre_moe"),
    ("fp8_decode", MOE_PATH_STREAM, "pre_moe"), ("int8_decode", MOE_PATH_STREAM, "pre_dense"),
    ("fp8_decode", MOE_PATH_STREAM, "pre_dense")])
def test_ffn_layer(dev, name, path, which):
    """moe_ffn_layer against the oracle's ffn_layer. Routing as in the block
    tests (on the residual h); the output compared whole and, since
    the residual dominates it, also minus h, with the rounding of the output
    to bf16 (half an ulp, 2^-9 relative) added to the bound."""
    wl, w, x, lw, xd = inputs(name, dev)
    s = wl.shape
    K, H = s.top_k, s.hidden
    say(f"case: ffn layer {name} path={path} norms={which}")
    norms_np, norms = ffn_gains(H, which, dev)
    T = xd.shape[0]
    out_t = dict(topk_idx=torch.empty((T, K), dtype=torch.int32, device=dev),
                 topk_w=torch.empty((T, K), dtype=torch.float32, device=dev))
    dbg = new_debug(path, **out_t)
    out = moe_ffn_layer(dims_of(s), lw, norms, xd, debug=dbg)
    torch.cuda.synchronize()
    assert dbg.path_taken == path
    toks = np.arange(T) if T <= FULL_CHECK_T else sample_tokens(T, n=64, seed=5)
    gi, gw = to_np(out_t["topk_idx"])[toks], to_np(out_t["topk_w"])[toks]
    ow, fmt = oracle_weights(wl, w)
    rel_max = REL_BF16 if fmt == "bf16" else REL_INT8
    _, ref_r = oracle.ffn_layer(x[toks], ow, norms_np, K, s.rms_eps, expert_dtype=fmt)
    check_routing(gi, gw, ref_r, w["per_expert_scale"])
    ref, _ = oracle.ffn_layer(x[toks], ow, norms_np, K, s.rms_eps, expert_dtype=fmt,
                              routing=routing_for(gi, ref_r, w["per_expert_scale"]))
    got = y_f64(out)[toks]
    h64 = oracle.bf16_to_f64(x[toks])
    compare_y(got, ref, rel_max)
    # the branches' part alone: its rel-L2 error may grow by the output's rounding
    # (2^-9 of |out| per element) and its cosine falls accordingly (1 - rel^2 / 2)
    branch_ref = ref - h64
    bound = rel_max + 2.0**-9 * np.linalg.norm(ref) / np.linalg.norm(branch_ref)
    a, b = (got - h64).ravel(), branch_ref.ravel()
    rel = float(np.linalg.norm(a - b) / np.linalg.norm(b))
    cos = float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))
    assert rel <= bound and cos >= 1.0 - bound * bound / 2, f"branches: rel-L2 {rel:.3g} (bound {bound:.3g}), cos {cos:.6f}"



CHUNK_CASES = [("tiny", 2048 + 77, 1024, None), ("tiny", 2048 + 20, 1500, "all"),
               ("long_prefill", None, 0, None), ("prefill", 2048 + 5, 1024, "all"),
               ("fp8_prefill", 2048 + 5, 1024, None)]


@pytest.mark.parametrize("name,T,chunk,which", CHUNK_CASES)
def test_prefill_chunked(dev, name, T, chunk, which):
    """moe_prefill_chunked: bit for bit the per-chunk calls of the block (or the
    layer), whose routing then serves the comparison with the oracle on sampled
    tokens, spread over every chunk. Chunks of 1024 tokens with a ragged last
    one of 77 or 5 tokens (the 5-token one takes the streaming path), 1500
    snapped down to 1024, and the real 40960-token prompt in the default
    16384-token chunks."""
    wl, w, x, lw, xd = inputs(name, dev, T)
    s = wl.shape
    T, K, H = x.shape[0], s.top_k, s.hidden
    C = moe_prefill_chunk_tokens(chunk)
    assert C == (16384 if chunk <= 0 else max(1024, min(32768, chunk // 1024 * 1024)))
    say(f"case: chunked prefill {name} T={T} chunk={C} norms={which}")
    norms_np, norms = ffn_gains(H, which, dev) if which else (None, None)
    ws = torch.empty(moe_prefill_workspace_bytes(dims_of(s), chunk), dtype=torch.uint8, device=dev)
    out = moe_prefill_chunked(dims_of(s), lw, norms, xd, chunk, workspace=ws)
    # the same chunks one call each, with their routing
    ref_out = torch.empty_like(out)
    gi = np.empty((T, K), np.int32)
    gw = np.empty((T, K), np.float32)
    for t0 in range(0, T, C):
        t1 = min(T, t0 + C)
        o = dict(topk_idx=torch.empty((t1 - t0, K), dtype=torch.int32, device=dev),
                 topk_w=torch.empty((t1 - t0, K), dtype=torch.float32, device=dev))
        dbg = new_debug(MOE_PATH_AUTO, **o)
        if norms is None:
            ref_out[t0:t1] = moe_block(dims_of(s), lw, xd[t0:t1], debug=dbg)
        else:
            ref_out[t0:t1] = moe_ffn_layer(dims_of(s), lw, norms, xd[t0:t1], debug=dbg)
        torch.cuda.synchronize()
        gi[t0:t1], gw[t0:t1] = to_np(o["topk_idx"]), to_np(o["topk_w"])
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), "chunked != per-chunk calls"
    toks = sample_tokens(T, n=64, seed=11)
    # the layer routes the residual h (the router normalises it itself)
    ow, fmt = oracle_weights(wl, w)
    ref_r = (oracle_route(wl, w, x[toks]) if norms is None
             else oracle.ffn_layer(x[toks], ow, norms_np, K, s.rms_eps, expert_dtype=fmt)[1])
    check_routing(gi[toks], gw[toks], ref_r, w["per_expert_scale"])
    r = routing_for(gi[toks], ref_r, w["per_expert_scale"])
    if norms is None:
        ref, _ = oracle.moe_block(x[toks], ow, K, s.rms_eps, expert_dtype=fmt, routing=r)
    else:
        ref, _ = oracle.ffn_layer(x[toks], ow, norms_np, K, s.rms_eps, expert_dtype=fmt, routing=r)
    cos, rel = compare_y(y_f64(out)[toks], ref, REL_BF16 if fmt == "bf16" else REL_INT8)
    say(f"  tokens checked {len(toks)}  cos {cos:.7f}  rel-L2 {rel:.3e}")


# ---------------------------------------------------------------- seeded random shapes
def _random_cases(n=8, seed=2024):
    """Small shapes drawn once from a fixed seed: hidden a multiple of 256 up to
    1024, 2..64 experts, top-k up to min(8, E), intermediates multiples of 64,
    ragged T from 1 to 300, each in the three expert formats."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        E = int(rng.integers(2, 65))
        shape = moe_synth.BlockShape(hidden=256 * int(rng.integers(1, 5)), num_experts=E,
                                     top_k=int(rng.integers(1, min(8, E) + 1)),
                                     expert_inter=64 * int(rng.integers(1, 5)),
                                     dense_inter=64 * int(rng.integers(1, 5)))
        T = int(rng.choice([1, 7, 33, 64, 65, 129, 300]))
        cases.append((i, shape, T, ("bf16", "int8", "fp8")[i % 3]))
    return cases


@pytest.mark.parametrize("case", _random_cases(), ids=lambda c: f"r{c[0]}-{c[3]}-T{c[2]}")
def test_random_shapes(dev, case):
    """moe_block on both paths (the streaming one where T <= 64) against the
    oracle on every token, at shapes none of the workloads has."""
    i, shape, T, fmt = case
    say(f"case: random shape {i}: {shape} T={T} experts {fmt}")
    w = moe_synth.make_weights(shape, 100 + i)
    x = moe_synth.make_tokens(shape, 100 + i, T)
    lw = upload(w, dev, int8=fmt == "int8", fp8=fmt == "fp8")
    xd = bf16_dev(x, dev)
    wl = moe_synth.Workload(f"random{i}", shape, T, 100 + i, int8=fmt == "int8", fp8=fmt == "fp8")
    ref_r = oracle_route(wl, w, x)
    ow, ofmt = oracle_weights(wl, w)
    paths = [MOE_PATH_GROUPED] + ([MOE_PATH_STREAM] if T <= 64 else [])
    for path in paths:
        y, dbg = run_block(wl, lw, xd, path)
        check_routing(dbg["topk_idx"], dbg["topk_w"], ref_r, w["per_expert_scale"])
        p = oracle.permute_pairs(dbg["topk_idx"], shape.num_experts)
        for k in ("counts", "offsets", "perm_token", "inv_row"):
            np.testing.assert_array_equal(dbg[k], p[k], err_msg=k)
        r = routing_for(dbg["topk_idx"], ref_r, w["per_expert_scale"])
        y_ref, _ = oracle.moe_block(x, ow, shape.top_k, shape.rms_eps, expert_dtype=ofmt, routing=r)
        cos, rel = compare_y(y_f64(y), y_ref, REL_BF16 if ofmt == "bf16" else REL_INT8)
        say(f"  path {path}: cos {cos:.7f}  rel-L2 {rel:.3e}")


@pytest.mark.parametrize("fmt", ["bf16", "int8", "fp8"])
@pytest.mark.parametrize("T", [5, 64])
def test_stream_many_rows(dev, fmt, T):
    """The streaming path with many rows per expert (8 experts, top-8: every
    expert takes every token), so that its staging of x, of h and of the
    dense rows runs over several passes of four rows, in each expert format,
    against the oracle on every token."""
    shape = EDGE["k_eq_e"]
    say(f"case: streaming, every expert takes all {T} tokens, experts {fmt}")
    w = moe_synth.make_weights(shape, 77)
    x = moe_synth.make_tokens(shape, 77, T)
    lw = upload(w, dev, int8=fmt == "int8", fp8=fmt == "fp8")
    wl = moe_synth.Workload("many_rows", shape, T, 77, int8=fmt == "int8", fp8=fmt == "fp8")
    ref_r = oracle_route(wl, w, x)
    ow, ofmt = oracle_weights(wl, w)
    y, dbg = run_block(wl, lw, bf16_dev(x, dev), MOE_PATH_STREAM)
    check_routing(dbg["topk_idx"], dbg["topk_w"], ref_r, w["per_expert_scale"])
    assert (dbg["counts"] == T).all()
    r = routing_for(dbg["topk_idx"], ref_r, w["per_expert_scale"])
    y_ref, _ = oracle.moe_block(x, ow, shape.top_k, shape.rms_eps, expert_dtype=ofmt, routing=r)
    rel_bar = REL_BF16 if ofmt == "bf16" else REL_INT8
    compare_y(y_f64(y), y_ref, rel_bar)
    compare_per_token(y_f64(y), y_ref, rel_bar)


@pytest.mark.parametrize("name", ["decode", "int8_decode", "fp8_decode"])
def test_stream_largest_batch_real_shape(dev, name):
    """The streaming path at its largest batch (T = 64) at the real shape, in
    each expert format: several rows per expert for most experts, so its
    staging runs over more than one pass, against the oracle on every token."""
    wl, w, x, lw, xd = inputs(name, dev, tokens=64)
    s = wl.shape
    say(f"case: streaming path, real shape, {name} weights, T=64")
    y, dbg = run_block(wl, lw, xd, MOE_PATH_STREAM)
    ref = oracle_route(wl, w, x)
    check_routing(dbg["topk_idx"], dbg["topk_w"], ref, w["per_expert_scale"])
    p = oracle.permute_pairs(dbg["topk_idx"], s.num_experts)
    for k in ("counts", "offsets", "perm_token", "inv_row"):
        np.testing.assert_array_equal(dbg[k], p[k], err_msg=k)
    assert int(dbg["counts"].max()) > 4  # at least one expert takes two passes
    r = routing_for(dbg["topk_idx"], ref, w["per_expert_scale"])
    ow, fmt = oracle_weights(wl, w)
    y_ref, _ = oracle.moe_block(x, ow, s.top_k, s.rms_eps, expert_dtype=fmt, routing=r)
    bar = REL_BF16 if fmt == "bf16" else REL_INT8
    cos, rel = compare_y(y_f64(y), y_ref, bar)
    worst = compare_per_token(y_f64(y), y_ref, bar)
    say(f"  cos {cos:.7f}  rel-L2 {rel:.3e}  worst token rel-L2 {worst:.3e}")
