"""Helpers for the GPU parity tests: upload seeded inputs, compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import moe_synth
import oracle
from mixture_experts_ffn_amd import BlockDims, LayerWeights, moe_quantize_fp8, moe_quantize_int8, tile_layer

COS_MIN = 0.9999
REL_BF16 = 1e-2
REL_INT8 = 2e-2
W_REL = 1e-5


def dims_of(shape: moe_synth.BlockShape) -> BlockDims:
    return BlockDims(shape.hidden, shape.num_experts, shape.top_k, shape.expert_inter,
                     shape.dense_inter, shape.rms_eps)


def bf16_dev(a: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)


def f32_dev(a, dev):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def upload(w: dict, dev, int8: bool = False, fp8: bool = False) -> LayerWeights:
    """Device copy of a generated layer, its expert and dense matrices in the
    tiled layout the block reads. int8 and E4M3 experts are quantised on the GPU
    by the library's own quantisers (row-major), then tiled."""
    gu = bf16_dev(w["expert_gate_up"], dev)
    dn = bf16_dev(w["expert_down"], dev)
    lw = LayerWeights(
        router_scale=bf16_dev(w["router_scale"], dev), router_w=bf16_dev(w["router_w"], dev),
        per_expert_scale=f32_dev(w["per_expert_scale"], dev), expert_gate_up=gu, expert_down=dn,
        dense_gate_up=bf16_dev(w["dense_gate_up"], dev), dense_down=bf16_dev(w["dense_down"], dev),
        logit_bias=f32_dev(w.get("logit_bias"), dev))
    if int8:
        lw.expert_gate_up, lw.gate_up_scale = moe_quantize_int8(gu)
        lw.expert_down, lw.down_scale = moe_quantize_int8(dn)
        del gu, dn
    if fp8:
        lw.expert_gate_up, lw.gate_up_scale = moe_quantize_fp8(gu)
        lw.expert_down, lw.down_scale = moe_quantize_fp8(dn)
        del gu, dn
    return tile_layer(lw)


def oracle_int8_weights(w: dict) -> dict:
    wq = dict(w)
    wq["expert_gate_up_q"], wq["expert_gate_up_scale"] = oracle.quantize_int8(w["expert_gate_up"])
    wq["expert_down_q"], wq["expert_down_scale"] = oracle.quantize_int8(w["expert_down"])
    return wq


def oracle_fp8_weights(w: dict) -> dict:
    wq = dict(w)
    wq["expert_gate_up_f8"], wq["expert_gate_up_f8_scale"] = oracle.quantize_fp8(w["expert_gate_up"])
    wq["expert_down_f8"], wq["expert_down_f8_scale"] = oracle.quantize_fp8(w["expert_down"])
    return wq


def oracle_weights(wl, w: dict):
    """(the oracle's weights, its expert_dtype) for a workload's format."""
    if wl.int8:
        return oracle_int8_weights(w), "int8"
    if wl.fp8:
        return oracle_fp8_weights(w), "fp8"
    return w, "bf16"


def check_routing(gpu_idx: np.ndarray, gpu_w: np.ndarray, ref: dict, pes: np.ndarray):
    """Indices bit-exact except on flagged near-ties; there, the GPU's set must
    also be a valid top-k within the tie band. Weights to W_REL relative,
    against the oracle's renormalised probabilities of the GPU's set."""
    K = gpu_idx.shape[1]
    flagged = ref["boundary_tie"] | ref["order_tie"]
    ok = ~flagged
    mism = np.where((gpu_idx[ok] != ref["topk_idx"][ok]).any(axis=1))[0]
    assert mism.size == 0, f"{mism.size} unflagged tokens differ, first {np.where(ok)[0][mism[:5]]}"
    for t in np.where(flagged)[0]:
        lg = ref["logits"][t]
        kth = np.sort(lg)[::-1][K - 1]
        assert len(set(gpu_idx[t].tolist())) == K
        assert (lg[gpu_idx[t]] >= kth - oracle.NEAR_TIE).all(), f"token {t}: invalid tie resolution"
    p = np.take_along_axis(ref["probs"], gpu_idx.astype(np.int64), axis=1)
    w_ref = p / p.sum(axis=1, keepdims=True) * pes.astype(np.float64)[gpu_idx]
    rel = np.abs(gpu_w - w_ref) / np.abs(w_ref)
    assert rel.max() <= W_REL, f"weights rel err {rel.max():.3g}"
    return int(flagged.sum())


def routing_for(gpu_idx: np.ndarray, ref: dict, pes: np.ndarray) -> dict:
    """Oracle routing that uses the GPU's index sets (identical to the oracle's
    except on flagged near-ties) with the oracle's fp64 weights."""
    p = np.take_along_axis(ref["probs"], gpu_idx.astype(np.int64), axis=1)
    return {"topk_idx": gpu_idx.astype(np.int32),
            "topk_w": p / p.sum(axis=1, keepdims=True) * pes.astype(np.float64)[gpu_idx]}


def compare_y(y_gpu: np.ndarray, y_ref: np.ndarray, rel_max: float):
    a = y_gpu.astype(np.float64).ravel()
    b = y_ref.astype(np.float64).ravel()
    cos = float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))
    rel = float(np.linalg.norm(a - b) / np.linalg.norm(b))
    assert cos >= COS_MIN and rel <= rel_max, f"cos {cos:.6f} rel-L2 {rel:.3g}"
    return cos, rel


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).cpu().numpy()
    return t.cpu().numpy()


def y_f64(t: torch.Tensor) -> np.ndarray:
    return oracle.bf16_to_f64(to_np(t))
