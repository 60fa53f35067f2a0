"""The seeded generator: determinism, bf16 rounding and shapes."""
import numpy as np

import moe_synth


def test_bf16_round_to_nearest_even():
    vals = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -1.0 - 2.0 ** -8,
                     1.0 + 2.0 ** -8 + 2.0 ** -20, 3.0e-39, 0.0, -0.0], dtype=np.float32)
    bits = moe_synth.f32_to_bf16_bits(vals)
    # 1+2^-8 is halfway between 1 and 1+2^-7: ties go to the even mantissa (1.0)
    assert bits.tolist() == [0x3F80, 0x3F80, 0x3F82, 0xBF80, 0x3F81,
                             moe_synth.f32_to_bf16_bits(np.array([3.0e-39], np.float32))[0], 0x0000, 0x8000]
    back = moe_synth.bf16_bits_to_f32(bits)
    assert back[0] == 1.0 and back[2] == np.float32(1.0 + 2.0 ** -6)


def test_bf16_rounding_error_bound():
    z = np.random.default_rng(0).standard_normal(100000).astype(np.float32)
    back = moe_synth.bf16_bits_to_f32(moe_synth.f32_to_bf16_bits(z))
    rel = np.abs(back - z) / np.abs(z)
    assert rel.max() <= 2.0 ** -8          # unit roundoff of an 8-bit significand


def test_generator_is_deterministic_and_weights_do_not_depend_on_T():
    wl = moe_synth.WORKLOADS["tiny"]
    a = moe_synth.make_weights(wl.shape, wl.seed)
    b = moe_synth.make_weights(wl.shape, wl.seed)
    for k in a:
        if a[k] is None:
            assert b[k] is None
        else:
            np.testing.assert_array_equal(a[k], b[k])
    x8 = moe_synth.make_tokens(wl.shape, wl.seed, 8)
    x64 = moe_synth.make_tokens(wl.shape, wl.seed, 64)
    np.testing.assert_array_equal(x8, x64[:8])


def test_shapes_and_distributions():
    wl, w, x = moe_synth.make_inputs("tiny")
    s = wl.shape
    assert x.shape == (64, s.hidden) and x.dtype == np.uint16
    assert w["expert_gate_up"].shape == (s.num_experts, 2 * s.expert_inter, s.hidden)
    assert w["expert_down"].shape == (s.num_experts, s.hidden, s.expert_inter)
    assert w["dense_gate_up"].shape == (2 * s.dense_inter, s.hidden)
    assert w["dense_down"].shape == (s.hidden, s.dense_inter)
    assert w["per_expert_scale"].dtype == np.float32
    assert (w["per_expert_scale"] >= 0.5).all() and (w["per_expert_scale"] <= 1.5).all()
    gu = moe_synth.bf16_bits_to_f32(w["expert_gate_up"])
    assert abs(gu.std() - 0.02) < 1e-3
    sc = moe_synth.bf16_bits_to_f32(w["router_scale"])
    assert abs(sc.mean() - 1.0) < 0.02 and abs(sc.std() - 0.1) < 0.02
    assert w["logit_bias"] is None


def test_skew_bias_is_zipf_log_rank():
    shp = moe_synth.BlockShape(hidden=256, num_experts=128, top_k=8, expert_inter=64, dense_inter=64)
    w = moe_synth.make_weights(shp, 3, skew=True)
    b = w["logit_bias"].astype(np.float64)
    ranks = np.sort(np.exp(-b / 1.2))
    np.testing.assert_allclose(ranks, np.arange(1, 129), rtol=1e-5)


def test_router_only_draw_matches_full_draw():
    shp = moe_synth.BlockShape(hidden=256, num_experts=16, top_k=4, expert_inter=64, dense_inter=64)
    full = moe_synth.make_weights(shp, 7, skew=True)
    ro = moe_synth.make_weights(shp, 7, skew=True, router_only=True)
    for k in ("router_scale", "router_w", "per_expert_scale", "logit_bias"):
        np.testing.assert_array_equal(full[k], ro[k])
    assert "expert_gate_up" not in ro
