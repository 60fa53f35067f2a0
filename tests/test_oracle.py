"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign, index or axis, a transposed operand, gate and up swapped) fails at
least one of them. None of them calls the HIP library.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import softmax as scipy_softmax

import moe_synth
from moe_synth import BlockShape
import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
SMALL = BlockShape(hidden=256, num_experts=8, top_k=3, expert_inter=64, dense_inter=128)


def _w64(w):
    """Weights dict with every bf16 tensor widened to float64 (for torch)."""
    return {k: (oracle.bf16_to_f64(v) if isinstance(v, np.ndarray) and v.dtype == np.uint16 else v)
            for k, v in w.items()}


@pytest.fixture(scope="module")
def tiny():
    return moe_synth.make_inputs("tiny")


# ---------------------------------------------------------------- GELU
def test_gelu_matches_torch_tanh_gelu():
    z = torch.linspace(-12, 12, 20001, dtype=torch.float64)
    ref = F.gelu(z, approximate="tanh").numpy()
    np.testing.assert_allclose(oracle.gelu_tanh(z.numpy()), ref, rtol=0, atol=1e-14)


def test_gelu_closed_forms():
    z = np.linspace(-5, 5, 1001)
    # 0.5 z (1 + t) - (-0.5 z (1 - t)) = z: the odd part of GELU is z / 2
    np.testing.assert_allclose(oracle.gelu_tanh(z) - oracle.gelu_tanh(-z), z, atol=1e-13)
    assert oracle.gelu_tanh(0.0) == 0.0
    assert abs(oracle.gelu_tanh(20.0) - 20.0) < 1e-12
    assert abs(oracle.gelu_tanh(-20.0)) < 1e-12
    c = math.sqrt(2 / math.pi)
    assert abs(oracle.gelu_tanh(1.0) - 0.5 * (1 + math.tanh(c * 1.044715))) < 1e-15


# ---------------------------------------------------------------- RMSNorm
def test_rmsnorm_identity():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 300)) * 3
    eps = 1e-6
    r = oracle.rms_normalise(x, eps)
    ms = np.mean(x * x, axis=1)
    np.testing.assert_allclose(np.mean(r * r, axis=1), ms / (ms + eps), rtol=1e-13)


# ---------------------------------------------------------------- router
def test_router_logits_closed_form():
    # one-hot router rows pick coordinates of v = x / rms(x) * s * H^-0.5
    H, E = 16, 4
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, H))
    s = 1 + 0.1 * rng.standard_normal(H)
    Wr = np.zeros((E, H))
    cols = [3, 0, 11, 7]
    for e, c in enumerate(cols):
        Wr[e, c] = 1.0
    got = oracle.router_logits(x, s, Wr, eps=0.0)
    rms = np.sqrt(np.mean(x * x, axis=1))
    want = np.stack([x[:, c] / rms * s[c] / math.sqrt(H) for c in cols], axis=1)
    np.testing.assert_allclose(got, want.astype(np.float32), rtol=1e-7)


def test_router_is_scale_free():
    _, w, x = moe_synth.make_inputs("tiny")
    x64 = oracle.bf16_to_f64(x)
    a = oracle.route(x64, w["router_scale"], w["router_w"], w["per_expert_scale"], 4, 0.0)
    b = oracle.route(4.0 * x64, w["router_scale"], w["router_w"], w["per_expert_scale"], 4, 0.0)
    np.testing.assert_array_equal(a["topk_idx"], b["topk_idx"])
    np.testing.assert_allclose(a["topk_w"], b["topk_w"], rtol=1e-12)


def test_router_renormalised_weights_sum_to_one(tiny):
    wl, w, x = tiny
    r = oracle.route(x, w["router_scale"], w["router_w"], w["per_expert_scale"], 4, 1e-6)
    np.testing.assert_allclose(r["renorm"].sum(axis=1), 1.0, atol=1e-12)
    pes = w["per_expert_scale"].astype(np.float64)[r["topk_idx"]]
    np.testing.assert_allclose((r["topk_w"] / pes).sum(axis=1), 1.0, atol=1e-12)
    # the per-expert scale multiplies the renormalised weight
    np.testing.assert_allclose(r["topk_w"], r["renorm"] * pes, rtol=1e-15)


def test_router_k_equals_e_is_full_softmax(tiny):
    wl, w, x = tiny
    E = w["router_w"].shape[0]
    r = oracle.route(x, w["router_scale"], w["router_w"], w["per_expert_scale"], E, 1e-6)
    full = scipy_softmax(r["logits"], axis=1)
    np.testing.assert_allclose(np.take_along_axis(full, r["topk_idx"].astype(np.int64), 1),
                               r["renorm"], rtol=1e-12)
    # every expert appears once
    np.testing.assert_array_equal(np.sort(r["topk_idx"], axis=1), np.tile(np.arange(E), (x.shape[0], 1)))


def test_router_selection_matches_library_topk(tiny):
    wl, w, x = tiny
    r = oracle.route(x, w["router_scale"], w["router_w"], w["per_expert_scale"], 4, 1e-6)
    assert not r["boundary_tie"].any() and not r["order_tie"].any()
    vals, idx = torch.topk(torch.from_numpy(r["logits"]), 4, dim=1, largest=True, sorted=True)
    np.testing.assert_array_equal(r["topk_idx"], idx.numpy())
    # softmax is monotone: selecting on probabilities gives the same set
    np.testing.assert_array_equal(np.sort(r["topk_idx"], 1),
                                  np.sort(np.argsort(-r["probs"], 1)[:, :4], 1))


def test_router_tie_goes_to_lower_index():
    H, E = 8, 6
    x = np.ones((1, H))
    Wr = np.zeros((E, H))
    Wr[[1, 2, 4, 5], 0] = 1.0           # experts 1, 2, 4, 5 tie; 0 and 3 lower
    Wr[3, 0] = -1.0
    r = oracle.route(x, np.ones(H), Wr, np.ones(E), 3, 0.0)
    np.testing.assert_array_equal(r["topk_idx"][0], [1, 2, 4])
    assert r["boundary_tie"][0] and r["order_tie"][0]
    np.testing.assert_allclose(r["renorm"][0], [1 / 3] * 3, rtol=1e-15)


def test_router_bias_is_added_to_logits():
    _, w, x = moe_synth.make_inputs("tiny")
    E = w["router_w"].shape[0]
    bias = np.zeros(E, dtype=np.float32)
    bias[5] = 100.0                      # forces expert 5 first for every token
    r = oracle.route(x, w["router_scale"], w["router_w"], w["per_expert_scale"], 4, 1e-6, bias)
    assert (r["topk_idx"][:, 0] == 5).all()
    r0 = oracle.route(x, w["router_scale"], w["router_w"], w["per_expert_scale"], 4, 1e-6)
    np.testing.assert_allclose(r["logits"][:, 5], (r0["logits"][:, 5] + 100.0).astype(np.float32),
                               rtol=1e-6)


# ---------------------------------------------------------------- permutation
def test_permutation_properties(tiny):
    wl, w, x = tiny
    r = oracle.route(x, w["router_scale"], w["router_w"], w["per_expert_scale"], 4, 1e-6)
    idx = r["topk_idx"]
    T, K = idx.shape
    E = 16
    p = oracle.permute_pairs(idx, E)
    assert p["counts"].sum() == T * K
    assert p["offsets"][0] == 0 and p["offsets"][-1] == T * K
    assert (np.diff(p["offsets"]) == p["counts"]).all()
    # bijection onto all pairs
    pairs = set(zip(p["perm_token"].tolist(), p["perm_slot"].tolist()))
    assert len(pairs) == T * K
    for e in range(E):
        a, b = p["offsets"][e], p["offsets"][e + 1]
        seg_t = p["perm_token"][a:b]
        assert (np.diff(seg_t) > 0).all()          # strictly increasing tokens
        assert (idx[seg_t, p["perm_slot"][a:b]] == e).all()
        # brute force: the tokens that picked e, in order
        want = [t for t in range(T) if e in idx[t]]
        assert seg_t.tolist() == want
    # inv_row is the inverse permutation
    rows = p["inv_row"]
    np.testing.assert_array_equal(p["perm_token"][rows], np.repeat(np.arange(T), K))
    np.testing.assert_array_equal(p["perm_slot"][rows], np.tile(np.arange(K), T))
    # a token never repeats an expert
    assert all(len(set(row)) == K for row in idx.tolist())


# ---------------------------------------------------------------- block
def test_masked_dense_equals_sparse_tiny(tiny):
    wl, w, x = tiny
    y_s, r = oracle.moe_block(x, w, 4, 1e-6)
    y_d, _ = oracle.masked_dense_block(x, w, 4, 1e-6, routing=r)
    np.testing.assert_allclose(y_d, y_s, rtol=1e-10, atol=1e-12)


def test_masked_dense_equals_sparse_real_width():
    # real hidden / intermediate widths, fewer experts to keep it fast
    shp = BlockShape(hidden=2816, num_experts=12, top_k=8, expert_inter=704, dense_inter=2112)
    w = moe_synth.make_weights(shp, 11)
    x = moe_synth.make_tokens(shp, 11, 6)
    y_s, r = oracle.moe_block(x, w, 8, 1e-6)
    y_d, _ = oracle.masked_dense_block(x, w, 8, 1e-6, routing=r)
    np.testing.assert_allclose(y_d, y_s, rtol=1e-9, atol=1e-12)


def test_single_expert_top1_reduces_to_dense_geglu():
    shp = BlockShape(hidden=128, num_experts=1, top_k=1, expert_inter=32, dense_inter=64)
    w = moe_synth.make_weights(shp, 3)
    x = moe_synth.make_tokens(shp, 3, 9)
    y, r = oracle.moe_block(x, w, 1, 1e-6)
    assert (r["topk_idx"] == 0).all()
    np.testing.assert_allclose(r["topk_w"][:, 0], w["per_expert_scale"][0], rtol=1e-15)
    # library reference: torch linear + tanh GELU (float64, CPU)
    w64 = _w64(w)
    xt = torch.from_numpy(oracle.bf16_to_f64(x))

    def geglu(gu, dn):
        gu = torch.from_numpy(gu)
        I = gu.shape[0] // 2
        h = F.gelu(F.linear(xt, gu[:I]), approximate="tanh") * F.linear(xt, gu[I:])
        return F.linear(h, torch.from_numpy(dn))

    want = float(w["per_expert_scale"][0]) * geglu(w64["expert_gate_up"][0], w64["expert_down"][0]) \
        + geglu(w64["dense_gate_up"], w64["dense_down"])
    np.testing.assert_allclose(y, want.numpy(), rtol=1e-10, atol=1e-12)


def test_dense_mlp_matches_torch():
    w = moe_synth.make_weights(SMALL, 4)
    x = moe_synth.make_tokens(SMALL, 4, 5)
    w64 = _w64(w)
    xt = torch.from_numpy(oracle.bf16_to_f64(x))
    gu = torch.from_numpy(w64["dense_gate_up"])
    Id = SMALL.dense_inter
    want = F.linear(F.gelu(F.linear(xt, gu[:Id]), approximate="tanh") * F.linear(xt, gu[Id:]),
                    torch.from_numpy(w64["dense_down"]))
    np.testing.assert_allclose(oracle.dense_mlp(x, w["dense_gate_up"], w["dense_down"]),
                               want.numpy(), rtol=1e-10, atol=1e-12)


def test_brute_force_loops_agree(tiny):
    wl, w, x = tiny
    toks = [0, 17, 63]
    y, _ = oracle.moe_block(x, w, 4, 1e-6)
    bf = oracle.brute_force_block(x, w, 4, 1e-6, toks)
    np.testing.assert_allclose(bf, y[toks], rtol=1e-10, atol=1e-12)


def test_tokens_are_independent(tiny):
    wl, w, x = tiny
    y, _ = oracle.moe_block(x, w, 4, 1e-6)
    for t in (0, 31, 63):
        yt, _ = oracle.moe_block(x[t:t + 1], w, 4, 1e-6)
        np.testing.assert_allclose(yt[0], y[t], rtol=1e-12, atol=1e-14)


def test_expert_relabelling_leaves_output_unchanged(tiny):
    wl, w, x = tiny
    y, r = oracle.moe_block(x, w, 4, 1e-6)
    assert not r["boundary_tie"].any()
    perm = np.random.default_rng(9).permutation(16)
    w2 = dict(w)
    for k in ("router_w", "per_expert_scale", "expert_gate_up", "expert_down"):
        w2[k] = w[k][perm]
    y2, r2 = oracle.moe_block(x, w2, 4, 1e-6)
    np.testing.assert_array_equal(perm[r2["topk_idx"]], r["topk_idx"])
    np.testing.assert_allclose(y2, y, rtol=1e-12, atol=1e-14)


def test_worked_example_closed_form():
    with open(os.path.join(HERE, "golden", "worked_example.json")) as f:
        ex = json.load(f)
    w = {k: np.array(ex[k], dtype=np.float64) for k in
         ("router_scale", "router_w", "per_expert_scale", "expert_gate_up", "expert_down",
          "dense_gate_up", "dense_down")}
    w["logit_bias"] = None
    x = np.array(ex["x"])

    def g(z):
        return 0.5 * z * (1 + math.tanh(math.sqrt(2 / math.pi) * (z + 0.044715 * z ** 3)))

    s1 = 1 / (1 + math.exp(-1))
    y1, r1 = oracle.moe_block(x, w, 1, ex["rms_eps"])
    np.testing.assert_array_equal(r1["topk_idx"], [[0]])
    np.testing.assert_allclose(r1["logits"], [[0.5, -0.5]], rtol=0)
    np.testing.assert_allclose(y1[0], [4 * g(1), -g(-1), 0, -4 * g(1)], rtol=1e-14, atol=1e-15)
    y2, r2 = oracle.moe_block(x, w, 2, ex["rms_eps"])
    np.testing.assert_array_equal(r2["topk_idx"], [[0, 1]])
    np.testing.assert_allclose(r2["topk_w"][0], [2 * s1, 3 * (1 - s1)], rtol=1e-14)
    want = (2 * s1 * np.array([2 * g(1), 0, 0, -2 * g(1)])
            + 3 * (1 - s1) * g(-1) * np.ones(4) + np.array([0, -g(-1), 0, 0]))
    np.testing.assert_allclose(y2[0], want, rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------- int8
def test_int8_quantisation_bounds():
    w = moe_synth.make_weights(SMALL, 6)
    q, s = oracle.quantize_int8(w["expert_gate_up"])
    assert q.dtype == np.int8 and s.dtype == np.float32
    wf = oracle.bf16_to_f64(w["expert_gate_up"])
    err = np.abs(wf - oracle.dequantize_int8(q, s))
    # nearest level: at most half a step, plus the rounding of the fp32 quotient
    # (half an ulp of a value below 128, i.e. 2^-18 of a step)
    assert (err <= s.astype(np.float64)[..., None] * (0.5 + 2.0 ** -18 + 1e-9)).all()
    assert (np.abs(q).max(axis=-1) == 127).all()
    assert (q != -128).all()


def test_int8_rounding_golden():
    # hand-picked row: max 127 -> scale 1; halves round to even; negative side symmetric
    row = np.array([[127.0, 2.5, 3.5, -2.5, -0.5, 0.49, 126.5, -127.0]], dtype=np.float32)
    q, s = oracle.quantize_int8(row)
    assert s[0] == np.float32(1.0)
    np.testing.assert_array_equal(q[0], [127, 2, 4, -2, 0, 0, 126, -127])
    zq, zs = oracle.quantize_int8(np.zeros((2, 5), dtype=np.float32))
    assert (zs == 0).all() and (zq == 0).all()


def test_int8_block_equals_block_on_dequantised_weights(tiny):
    wl, w, x = tiny
    wq = dict(w)
    wq["expert_gate_up_q"], wq["expert_gate_up_scale"] = oracle.quantize_int8(w["expert_gate_up"])
    wq["expert_down_q"], wq["expert_down_scale"] = oracle.quantize_int8(w["expert_down"])
    y8, r = oracle.moe_block(x, wq, 4, 1e-6, expert_dtype="int8")
    wd = dict(w)
    wd["expert_gate_up"] = oracle.dequantize_int8(wq["expert_gate_up_q"], wq["expert_gate_up_scale"])
    wd["expert_down"] = oracle.dequantize_int8(wq["expert_down_q"], wq["expert_down_scale"])
    yd, _ = oracle.moe_block(x, wd, 4, 1e-6, routing=r)
    np.testing.assert_allclose(y8, yd, rtol=1e-12, atol=1e-14)
    # and it stays close to the bf16 block (per-channel int8 loses little)
    yb, _ = oracle.moe_block(x, w, 4, 1e-6, routing=r)
    rel = np.linalg.norm(y8 - yb) / np.linalg.norm(yb)
    assert rel < 2e-2


# ---------------------------------------------------------------- fp8 (E4M3)
# the vLLM recipe page ("Gemma 4 26B-A4B IT"), variants > fp8: E4M3 weights,
# dynamic per-token activation quantisation


def _fp8_table():
    """Every finite E4M3 code and its value, built from numpy's float16: an
    E4M3 code's bits placed at the top of a float16 (sign at bit 15, exponent
    and mantissa at bits 7..13) are that code's value times 2^-8, subnormals
    included (the two formats' exponent biases differ by 8)."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    c = codes.astype(np.uint16)
    h = (((c & 0x80) << 8) | ((c & 0x7F) << 7)).astype(np.uint16).view(np.float16)
    return codes, h.astype(np.float64) * 256.0


def test_fp8_decode_against_float16_placement():
    codes, vals = _fp8_table()
    np.testing.assert_array_equal(oracle.fp8_e4m3_decode(codes), vals)
    assert oracle.fp8_e4m3_decode(np.array([0x7E]))[0] == 448.0
    assert oracle.fp8_e4m3_decode(np.array([0x01]))[0] == 2.0 ** -9
    assert np.isnan(oracle.fp8_e4m3_decode(np.array([0x7F, 0xFF]))).all()


def test_fp8_encode_golden():
    v = np.array([0.0, -0.0, 1.0, -2.0, 448.0, 2.0 ** -9, 2.0 ** -6, 7 * 2.0 ** -9,
                  1.0625, 1.1875, 1.125, 464.0, 500.0, 2.0 ** -10, 1.5 * 2.0 ** -9], dtype=np.float32)
    # 1.0625, 1.1875, 464, 2^-10 and 1.5 2^-9 lie halfway: ties go to the even code
    want = [0x00, 0x80, 0x38, 0xC0, 0x7E, 0x01, 0x08, 0x07, 0x38, 0x3A, 0x39, 0x7E, 0x7E, 0x00, 0x02]
    assert oracle.fp8_e4m3_encode(v).tolist() == want


def test_fp8_encode_is_nearest_by_brute_force():
    """Against a search over every finite value: the nearest, ties to the even
    code (magnitudes up to 464, the midpoint past 448)."""
    codes, vals = _fp8_table()
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.uniform(-464, 464, 4000), rng.uniform(-0.02, 0.02, 4000),
                        vals[np.isfinite(vals)], (vals[:-1] + vals[1:]) / 2]).astype(np.float32)
    got = oracle.fp8_e4m3_encode(v)
    dist = np.abs(vals[None, :] - v.astype(np.float64)[:, None])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    for i in range(v.size):
        c = codes[cand[i]]
        if c.size > 1:   # a tie: the even mantissa (for +-0 the sign of v)
            c = c[(c & 1) == 0]
            if c.size > 1:
                c = c[(c >> 7) == np.signbit(v[i])]
        assert got[i] == c[0], (v[i], got[i], c)


def test_fp8_quantisation_bounds():
    rng = np.random.default_rng(4)
    w = moe_synth.f32_to_bf16_bits((0.02 * rng.standard_normal((64, 256))).astype(np.float32))
    q, s = oracle.quantize_fp8(w)
    w64 = oracle.bf16_to_f64(w)
    amax = np.abs(w64).max(axis=1)
    np.testing.assert_array_equal(s, (amax.astype(np.float32) / np.float32(448)).astype(np.float32))
    dq = oracle.dequantize_fp8(q, s)
    # the largest element lands on +-448 scale; every element within half a step
    # (2^-4 relative for normals, 2^-10 scale below 2^-6 scale)
    assert np.all(np.abs(oracle.fp8_e4m3_decode(q)).max(axis=1) == 448.0)
    step = np.maximum(np.abs(dq) * 2.0 ** -4, 2.0 ** -10 * s[:, None])
    assert np.all(np.abs(dq - w64) <= step * (1 + 1e-6))
    zq, zs = oracle.quantize_fp8(np.zeros((2, 5), dtype=np.float32))
    assert (zs == 0).all() and (zq == 0).all()


def _fp8_weights(w):
    wq = dict(w)
    wq["expert_gate_up_f8"], wq["expert_gate_up_f8_scale"] = oracle.quantize_fp8(w["expert_gate_up"])
    wq["expert_down_f8"], wq["expert_down_f8_scale"] = oracle.quantize_fp8(w["expert_down"])
    return wq


def test_fp8_block_sparse_equals_masked_dense_and_tracks_bf16(tiny):
    wl, w, x = tiny
    wq = _fp8_weights(w)
    y8, r = oracle.moe_block(x, wq, 4, 1e-6, expert_dtype="fp8")
    ym, _ = oracle.masked_dense_block(x, wq, 4, 1e-6, expert_dtype="fp8", routing=r)
    np.testing.assert_allclose(y8, ym, rtol=1e-12, atol=1e-13)
    # quantisation noise of three 3-bit-mantissa roundings: visible, but small
    yb, _ = oracle.moe_block(x, w, 4, 1e-6, routing=r)
    yd = oracle.dense_mlp(x, w["dense_gate_up"], w["dense_down"])
    rel = np.linalg.norm((y8 - yd) - (yb - yd)) / np.linalg.norm(yb - yd)
    assert 1e-3 < rel < 0.12, rel


def test_fp8_expert_activation_quantisation_is_per_token(tiny):
    """Each token's row is quantised on its own: a token's output does not
    depend on the other rows, and scaling a row by a power of two scales its
    quantised input exactly (the codes stay, the scale doubles)."""
    wl, w, x = tiny
    wq = _fp8_weights(w)
    e = 3
    args = (wq["expert_gate_up_f8"][e], wq["expert_gate_up_f8_scale"][e],
            wq["expert_down_f8"][e], wq["expert_down_f8_scale"][e])
    rows = oracle.bf16_to_f64(x[:6])
    full = oracle.expert_ffn_fp8(rows, *args)
    for t in (0, 5):
        np.testing.assert_allclose(oracle.expert_ffn_fp8(rows[t:t + 1], *args)[0], full[t], rtol=1e-12, atol=1e-15)
    q1, s1 = oracle.quantize_fp8(rows.astype(np.float32))
    q2, s2 = oracle.quantize_fp8((2 * rows).astype(np.float32))
    np.testing.assert_array_equal(q1, q2)
    np.testing.assert_array_equal(s2, 2 * s1)


def test_fp8_expert_golden():
    """A hand-derived fp8 expert (tests/golden/fp8_expert.json): the codes of x
    and of the weights, and the output, which depends on h being rounded to
    bf16 and then quantised per row (the fixture records what either slip
    would give instead)."""
    with open(os.path.join(HERE, "golden", "fp8_expert.json")) as f:
        ex = json.load(f)
    x = np.array(ex["x"], dtype=np.float32)
    gu = np.array(ex["gate_up"], dtype=np.float32)
    dn = np.array(ex["down"], dtype=np.float32)
    xq, xs = oracle.quantize_fp8(x)
    np.testing.assert_array_equal(xq[0], ex["x_codes"])
    assert xs[0] == ex["scale"]
    guq, gus = oracle.quantize_fp8(gu)
    np.testing.assert_array_equal(guq, ex["gate_up_codes"])
    assert (gus == ex["scale"]).all()
    dnq, dns = oracle.quantize_fp8(dn)
    np.testing.assert_array_equal(dns, [ex["scale"], ex["scale"], 0.0, 0.0, 0.0])
    y = oracle.expert_ffn_fp8(x, guq, gus, dnq, dns)
    np.testing.assert_array_equal(y[0], ex["expected_y"])
    assert not np.array_equal(ex["expected_y"], ex["if_h_not_rounded_to_bf16"])
    assert not np.array_equal(ex["expected_y"], ex["if_h_not_quantised"])


# ---------------------------------------------------------------- accumulation
def test_fp16_accumulation_loses_accuracy_at_real_hidden():
    """Negative control for the ONNX export card, "MoE dispatch: why this
    export uses the vectorized unfused path": accumulating the expert products
    in fp16 at hidden 2816 is far less accurate than accumulating in fp32."""
    shp = BlockShape(hidden=2816, num_experts=1, top_k=1, expert_inter=64, dense_inter=64)
    w = moe_synth.make_weights(shp, 8)
    x = oracle.bf16_to_f64(moe_synth.make_tokens(shp, 8, 4))
    gate = oracle.bf16_to_f64(w["expert_gate_up"][0][:64])
    exact = x @ gate.T
    prod16 = (x[:, None, :] * gate[None, :, :]).astype(np.float16)
    acc16 = np.zeros(exact.shape, dtype=np.float16)
    acc32 = np.zeros(exact.shape, dtype=np.float32)
    for h in range(2816):                        # sequential accumulation
        acc16 = (acc16 + prod16[:, :, h]).astype(np.float16)
        acc32 = (acc32 + prod16[:, :, h].astype(np.float32)).astype(np.float32)
    e16 = np.linalg.norm(acc16 - exact) / np.linalg.norm(exact)
    e32 = np.linalg.norm(acc32 - exact) / np.linalg.norm(exact)
    assert e16 > 10 * e32


# ---------------------------------------------------------------- the layer's FFN (norms, residual)
NO_NORMS = {**dict.fromkeys(oracle.FFN_NORMS), "eps": 1e-6}


def test_rms_norm_scaled_invariants():
    rng = np.random.default_rng(5)
    v = rng.standard_normal((6, 256)) * rng.uniform(0.1, 10.0, (6, 1))
    s = 1.0 + 0.1 * rng.standard_normal(256)
    ones = np.ones(256)
    # invariant under scaling the row (eps = 0)
    np.testing.assert_allclose(oracle.rms_norm_scaled(3.7 * v, s, 0.0), oracle.rms_norm_scaled(v, s, 0.0),
                               rtol=1e-13)
    # unit gain: the output's mean square is ms / (ms + eps), in closed form
    eps = 0.25
    ms = np.mean(v * v, axis=1)
    out = oracle.rms_norm_scaled(v, ones, eps)
    np.testing.assert_allclose(np.mean(out * out, axis=1), ms / (ms + eps), rtol=1e-13)
    # unit gain, eps = 0: normalising a normalised row changes nothing
    n1 = oracle.rms_norm_scaled(v, ones, 0.0)
    np.testing.assert_allclose(oracle.rms_norm_scaled(n1, ones, 0.0), n1, rtol=1e-13)
    # the gain scales channels (columns), not tokens
    np.testing.assert_allclose(oracle.rms_norm_scaled(v, s, 0.0), n1 * s[None, :], rtol=1e-13)
    # no gain: no norm at that position
    assert np.array_equal(oracle.rms_norm_scaled(v, None, 0.5), v)


def test_round_bf16_ties_to_even_and_generator_agreement():
    v = np.array([1.0, 1 + 2.0**-8, 1 + 3 * 2.0**-8, -(1 + 2.0**-8), 2.5])
    np.testing.assert_array_equal(oracle.round_bf16(v), [1.0, 1.0, 1 + 2.0**-6, -1.0, 2.5])
    r = np.random.default_rng(1).standard_normal(20000).astype(np.float32)
    np.testing.assert_array_equal(oracle.round_bf16(r),
                                  moe_synth.bf16_bits_to_f32(moe_synth.f32_to_bf16_bits(r)).astype(np.float64))


def test_ffn_layer_without_norms_is_residual_plus_block(tiny):
    wl, w, x = tiny
    y, r = oracle.moe_block(x, w, wl.shape.top_k, wl.shape.rms_eps)
    out, _ = oracle.ffn_layer(x, w, NO_NORMS, wl.shape.top_k, wl.shape.rms_eps, routing=r)
    np.testing.assert_array_equal(out, oracle.bf16_to_f64(x) + y)


def test_ffn_layer_equal_pre_norms_feed_both_branches(tiny):
    """Equal pre-norm gains on both branches: the layer is the residual plus
    the block run on the normalised input rounded to bf16, routed on the
    residual h itself."""
    wl, w, x = tiny
    K, eps = wl.shape.top_k, wl.shape.rms_eps
    g = oracle.round_bf16(1.0 + 0.1 * np.random.default_rng(2).standard_normal(wl.shape.hidden))
    norms = {**NO_NORMS, "pre_dense": g, "pre_moe": g, "eps": 1e-5}
    out, r = oracle.ffn_layer(x, w, norms, K, eps)
    r_ref = oracle.route(x, w["router_scale"], w["router_w"], w["per_expert_scale"], K, eps)
    np.testing.assert_array_equal(r["topk_idx"], r_ref["topk_idx"])
    np.testing.assert_array_equal(r["topk_w"], r_ref["topk_w"])
    xn = oracle.round_bf16(oracle.rms_normalise(x, 1e-5) * g[None, :])
    y, _ = oracle.moe_block(xn, w, K, eps, routing=r)
    np.testing.assert_array_equal(out, oracle.bf16_to_f64(x) + y)


def test_ffn_layer_routing_ignores_the_pre_norms(tiny):
    """The router reads the un-normalised residual: its choice and weights do
    not move with the pre-norm gains, while the MoE branch's output does; and
    since the router's own norm is scale-free, scaling h by a power of two
    leaves the routing unchanged."""
    wl, w, x = tiny
    K, eps = wl.shape.top_k, wl.shape.rms_eps
    H = wl.shape.hidden
    rng = np.random.default_rng(12)
    g1 = oracle.round_bf16(1.0 + 0.3 * rng.standard_normal(H))
    g2 = oracle.round_bf16(1.0 + 0.3 * rng.standard_normal(H))
    a, ra = oracle.ffn_layer(x, w, {**NO_NORMS, "pre_moe": g1}, K, eps)
    b, rb = oracle.ffn_layer(x, w, {**NO_NORMS, "pre_moe": g2}, K, eps)
    np.testing.assert_array_equal(ra["topk_idx"], rb["topk_idx"])
    np.testing.assert_array_equal(ra["topk_w"], rb["topk_w"])
    assert np.max(np.abs(a - b)) > 1e-3
    _, r4 = oracle.ffn_layer(oracle.bf16_to_f64(x) * 4.0, w, {**NO_NORMS, "pre_moe": g1}, K, 0.0)
    _, r1 = oracle.ffn_layer(x, w, {**NO_NORMS, "pre_moe": g1}, K, 0.0)
    np.testing.assert_array_equal(r4["topk_idx"], r1["topk_idx"])


def test_ffn_layer_moe_branch_alone(tiny):
    """No dense weights, unit post gains and eps 0: the dense branch adds
    nothing and the outer norm of an already normalised row changes nothing,
    so the layer is h + N(moe(h))."""
    wl, w, x = tiny
    K, eps = wl.shape.top_k, wl.shape.rms_eps
    w0 = dict(w)
    w0["dense_gate_up"] = np.zeros_like(w["dense_gate_up"])
    w0["dense_down"] = np.zeros_like(w["dense_down"])
    ones = np.ones(wl.shape.hidden)
    norms = {**NO_NORMS, "post_moe": ones, "post": ones, "eps": 0.0}
    out, r = oracle.ffn_layer(x, w0, norms, K, eps)
    moe, _ = oracle.moe_part(x, w0, K, eps, routing=r)
    np.testing.assert_allclose(out, oracle.bf16_to_f64(x) + oracle.rms_normalise(moe, 0.0), rtol=1e-12,
                               atol=1e-12)


def test_ffn_layer_post_norms_act_per_branch(tiny):
    """Scaling the dense branch's down matrix by c > 0 leaves its post-normed
    output (eps 0) unchanged; without that norm the layer changes."""
    wl, w, x = tiny
    K, eps = wl.shape.top_k, wl.shape.rms_eps
    H = wl.shape.hidden
    w2 = dict(w)
    w2["dense_down"] = oracle.bf16_to_f64(w["dense_down"]) * 4.0  # exact: a power of two
    g = 1.0 + 0.1 * np.random.default_rng(3).standard_normal(H)
    with_norm = {**NO_NORMS, "post_dense": g, "post_moe": g, "post": g, "eps": 0.0}
    a, r = oracle.ffn_layer(x, w, with_norm, K, eps)
    b, _ = oracle.ffn_layer(x, w2, with_norm, K, eps, routing=r)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)
    c, _ = oracle.ffn_layer(x, w, NO_NORMS, K, eps, routing=r)
    d, _ = oracle.ffn_layer(x, w2, NO_NORMS, K, eps, routing=r)
    assert np.max(np.abs(c - d)) > 1e-3


def test_ffn_layer_pre_norms_act_per_branch(tiny):
    """A pre-norm on the MoE branch only: the experts read the normalised
    input, the dense MLP and the router the raw one."""
    wl, w, x = tiny
    K, eps = wl.shape.top_k, wl.shape.rms_eps
    g = oracle.round_bf16(1.0 + 0.1 * np.random.default_rng(4).standard_normal(wl.shape.hidden))
    out, r = oracle.ffn_layer(x, w, {**NO_NORMS, "pre_moe": g}, K, eps)
    xn = oracle.round_bf16(oracle.rms_normalise(x, 1e-6) * g[None, :])
    moe, _ = oracle.moe_part(xn, w, K, eps, routing=r)
    dense = oracle.dense_mlp(x, w["dense_gate_up"], w["dense_down"])
    np.testing.assert_array_equal(out, oracle.bf16_to_f64(x) + (dense + moe))
    r_ref = oracle.route(x, w["router_scale"], w["router_w"], w["per_expert_scale"], K, eps)
    np.testing.assert_array_equal(r["topk_idx"], r_ref["topk_idx"])
