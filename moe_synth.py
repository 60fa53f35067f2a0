"""Seeded synthetic inputs for the hybrid MoE FFN block.

This module only draws random numbers and stores them; it holds none of the
block's arithmetic. Both the CPU oracle and the GPU tests/bench take their
inputs from here, so the two sides always see the same bytes.

Shapes follow the Gemma-4 26B-A4B block as the pages describe it (Inferentia2
bf16 model card, "The architecture (a dual-path FFN)"; ONNX fp16 export card,
"Truthful graph contracts", rows "Mixture of Experts" and "Router"):
hidden 2816, 128 experts, top-8, expert intermediate 704, dense intermediate
2112. No real weights are available, so every tensor is a seeded draw.

Recipe (per workload seed ``s``):

* ``SeedSequence(s).spawn(3)`` gives three independent PCG64 streams: stream 0
  draws the weights, stream 1 the activations, stream 2 the skew permutation.
  The weights of a workload thus do not depend on how many tokens are drawn,
  and the router weights can be drawn without the experts.
* Weight stream, in this order, all drawn as float32 and then rounded to
  bfloat16 with round-to-nearest-even unless noted:
  router scale ``1 + 0.1*N(0,1)`` [H]; router weight ``0.02*N`` [E,H];
  per-expert scale ``U(0.5,1.5)`` [E] (kept float32); expert gate_up
  ``0.02*N`` [E,2I,H] drawn expert by expert; expert down ``0.02*N`` [E,H,I]
  expert by expert; dense gate_up ``0.02*N`` [2Id,H]; dense down ``0.02*N``
  [H,Id].
* Skew stream (skewed workload only): ``perm = permutation(E)`` and a logit
  bias ``-1.2*ln(perm+1)`` (float32), i.e. the log-probability of a Zipf law
  with exponent 1.2 over a random rank order.
* Activation stream: ``x = N(0,1)`` [T,H], rounded to bfloat16.

Rows ``[0, I)`` of a gate_up matrix are the gate projection and rows
``[I, 2I)`` the up projection (the same convention for the dense MLP with Id).
bfloat16 tensors are returned as ``uint16`` bit patterns.
"""
from __future__ import annotations

import dataclasses

import numpy as np

__all__ = ["BlockShape", "WORKLOADS", "Workload", "f32_to_bf16_bits",
           "bf16_bits_to_f32", "make_weights", "make_tokens", "make_inputs"]


@dataclasses.dataclass(frozen=True)
class BlockShape:
    hidden: int
    num_experts: int
    top_k: int
    expert_inter: int
    dense_inter: int
    rms_eps: float = 1e-6


REAL = BlockShape(hidden=2816, num_experts=128, top_k=8, expert_inter=704, dense_inter=2112)
TINY = BlockShape(hidden=512, num_experts=16, top_k=4, expert_inter=128, dense_inter=384)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shape: BlockShape
    tokens: int
    seed: int
    skew: bool = False
    int8: bool = False
    fp8: bool = False
    note: str = ""


WORKLOADS = {
    "tiny": Workload("tiny", TINY, 64, 0, note="plumbing case the oracle finishes in seconds"),
    "decode": Workload("decode", REAL, 8, 1, note="one real-shape layer, decode T=8"),
    "prefill": Workload("prefill", REAL, 2048, 2, note="real shape, T=2048, balanced routing"),
    "skew": Workload("skew", REAL, 16384, 3, skew=True,
                     note="real shape, one 16384-token chunk, Zipf(1.2) logit bias"),
    "int8_decode": Workload("int8_decode", REAL, 8, 4, int8=True,
                            note="real shape, int8 per-channel experts, T=8"),
    "int8_prefill": Workload("int8_prefill", REAL, 4096, 4, int8=True,
                             note="real shape, int8 per-channel experts, T=4096"),
    "fp8_decode": Workload("fp8_decode", REAL, 8, 5, fp8=True,
                           note="real shape, E4M3 experts with per-token activation quantisation, T=8"),
    "fp8_prefill": Workload("fp8_prefill", REAL, 2048, 5, fp8=True,
                            note="real shape, E4M3 experts with per-token activation quantisation, T=2048"),
    "mtp_decode": Workload("mtp_decode", REAL, 40, 1,
                           note="real shape, multi-token decode: 8 sequences x 5 tokens"),
    "long_prefill": Workload("long_prefill", REAL, 40960, 2,
                             note="real shape, a 40960-token prompt prefilled in 16384-token chunks"),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _streams(seed: int):
    return [np.random.Generator(np.random.PCG64(c)) for c in np.random.SeedSequence(seed).spawn(3)]


def _normal_bf16(rng, shape, std, mean=0.0):
    z = rng.standard_normal(shape, dtype=np.float32)
    z *= np.float32(std)
    if mean:
        z += np.float32(mean)
    return f32_to_bf16_bits(z)


def make_weights(shape: BlockShape, seed: int, skew: bool = False, router_only: bool = False) -> dict:
    """Draw one layer's weights (see the module docstring for the recipe).

    ``router_only`` stops after the router tensors (and the skew bias)."""
    rng, _, rng_skew = _streams(seed)
    H, E, I, Id = shape.hidden, shape.num_experts, shape.expert_inter, shape.dense_inter
    w = {}
    w["router_scale"] = _normal_bf16(rng, (H,), 0.1, mean=1.0)
    w["router_w"] = _normal_bf16(rng, (E, H), 0.02)
    w["per_expert_scale"] = rng.uniform(0.5, 1.5, size=(E,)).astype(np.float32)
    if skew:
        perm = rng_skew.permutation(E)
        w["logit_bias"] = (-1.2 * np.log(perm.astype(np.float64) + 1.0)).astype(np.float32)
    else:
        w["logit_bias"] = None
    if router_only:
        return w
    gu = np.empty((E, 2 * I, H), dtype=np.uint16)
    for e in range(E):
        gu[e] = _normal_bf16(rng, (2 * I, H), 0.02)
    w["expert_gate_up"] = gu
    dn = np.empty((E, H, I), dtype=np.uint16)
    for e in range(E):
        dn[e] = _normal_bf16(rng, (H, I), 0.02)
    w["expert_down"] = dn
    w["dense_gate_up"] = _normal_bf16(rng, (2 * Id, H), 0.02)
    w["dense_down"] = _normal_bf16(rng, (H, Id), 0.02)
    return w


def make_tokens(shape: BlockShape, seed: int, tokens: int) -> np.ndarray:
    """Draw the activations x [T, H] as bfloat16 bits."""
    rng = _streams(seed)[1]
    return _normal_bf16(rng, (tokens, shape.hidden), 1.0)


def make_inputs(workload: str | Workload, tokens: int | None = None):
    """Return ``(workload, weights, x)`` for a named workload."""
    wl = WORKLOADS[workload] if isinstance(workload, str) else workload
    T = wl.tokens if tokens is None else tokens
    return wl, make_weights(wl.shape, wl.seed, wl.skew), make_tokens(wl.shape, wl.seed, T)
