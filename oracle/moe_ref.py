"""Plain, slow CPU oracle of the Gemma-4 26B-A4B hybrid MoE FFN block.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; the product path never uses it.
It shares no code with the HIP library: it reads the seeded inputs (bfloat16
bit patterns) and nothing else.

Pages this follows (titles as printed on them):

* [INF2]  "Gemma-4 26B-A4B (MoE) on AWS Inferentia2 -- Tensor-Parallel (TP=8)"
* [INT8]  "Gemma-4 26B-A4B (MoE, int8 experts) on AWS Inferentia2 -- TP=8"
* [TT]    "Gemma-4-26B-A4B-it -- Tenstorrent Blackhole (vLLM bundle)"
* [ONNX]  "Gemma-4 26B-A4B-it -- ONNX MoE text decoder (fp16, CUDA) with
  canonical inference metadata"

What the block computes (one input x feeds router, experts and dense MLP):

* Router -- [ONNX] "Truthful graph contracts", row "Router": a scale-free
  RMSNorm, a learned scale times hidden^-0.5, a linear map to one logit per
  expert, a softmax in fp32, top-8, renormalisation of the 8 weights, then the
  per-expert scale.
* Experts -- [INF2] "The architecture (a dual-path FFN)" (128 experts, top 8,
  expert intermediate 704, hidden 2816) and [ONNX] row "Mixture of Experts"
  (activation ``gelu_pytorch_tanh``); [INF2] "How it works (the recipe)" maps
  each expert onto a fused gate_up linear and a down linear.
* Block output -- [ONNX] row "MoE topology": a dense MLP (intermediate 2112)
  in parallel with the MoE; the block result here is ``dense(x) + moe(x)``.
  ``ffn_layer`` adds the norms and the residual around it (see there).
* Sparse top-8 equals all-experts-dense with zero weight on the unselected
  experts -- [INF2] "How it works (the recipe)", first bullet.
* int8 experts -- [INT8] intro and "How it works": per-channel symmetric int8
  expert weights, every other weight bf16.
* fp8 experts -- the vLLM recipe page ("Gemma 4 26B-A4B IT"), ``variants`` ›
  fp8: E4M3 expert weights with dynamic per-token activation quantisation.

Precision. Everything is float64 except where the pages fix a precision: the
router's softmax works on fp32 logits ([ONNX] row "Router"), so the logits are
rounded to fp32 before the selection and the softmax (the softmax itself is
then evaluated exactly, in float64, on those fp32 values). The int8 quantiser
runs in fp32, the precision the GPU quantiser uses, so both take the same
integer decisions.

Readings where the pages are silent:
RMSNorm is ``x / sqrt(mean(x^2) + eps)`` with eps inside the root; the learned
scale is a per-channel vector; top-k selects by logit, descending, ties going
to the lower expert index, and emits the experts in that order; gate rows come
before up rows in a gate_up matrix; the dense MLP has the same GeGLU form as an
expert; int8 scales are per output channel, ``max|w|/127``, rounding half to
even. fp8: E4M3 in its OCP form without infinities (bias 7, largest finite
448); weight scales per output channel and activation scales per token (per
row of each expert linear's input), both ``amax/448`` in fp32, codes rounded
half to even in fp32; the expert's h is quantised from its bf16 value (the
activations between operators of a bf16 model are bf16 tensors); router and
dense MLP stay bf16. In the layer (``ffn_layer``) the router reads the
un-normalised residual stream, the experts their branch's pre-normed input.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "bf16_to_f64", "gelu_tanh", "rms_normalise", "router_logits", "route",
    "permute_pairs", "expert_ffn", "dense_mlp", "moe_part", "moe_block", "masked_dense_block",
    "quantize_int8", "dequantize_int8", "brute_force_block", "NEAR_TIE",
    "round_bf16", "rms_norm_scaled", "FFN_NORMS", "ffn_layer",
    "FP8_MAX", "fp8_e4m3_encode", "fp8_e4m3_decode", "quantize_fp8", "dequantize_fp8", "expert_ffn_fp8",
]

#: logit gap under which a top-k decision is reported as a near-tie
NEAR_TIE = 1e-6


def bf16_to_f64(bits) -> np.ndarray:
    """Exact value of bfloat16 bit patterns, as float64."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _f64(a):
    """Inputs arrive as bfloat16 bits (uint16) or as plain floats."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_to_f64(a)
    return a.astype(np.float64)


# --------------------------------------------------------------------------
# activation: [ONNX] "Truthful graph contracts", row "Mixture of Experts"
# names gelu_pytorch_tanh, the tanh approximation of GELU (Hendrycks & Gimpel,
# "Gaussian Error Linear Units", 2016): 0.5 z (1 + tanh(sqrt(2/pi)(z + 0.044715 z^3))).
# --------------------------------------------------------------------------
def gelu_tanh(z):
    z = np.asarray(z, dtype=np.float64)
    c = math.sqrt(2.0 / math.pi)
    return 0.5 * z * (1.0 + np.tanh(c * (z + 0.044715 * z * z * z)))


# --------------------------------------------------------------------------
# router: [ONNX] "Truthful graph contracts", row "Router"
# --------------------------------------------------------------------------
def rms_normalise(x, eps):
    """Scale-free RMSNorm: each token divided by its root-mean-square (no gain)."""
    x = _f64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps)


def router_logits(x, router_scale, router_w, eps, logit_bias=None):
    """Logits [T, E]: RMSNorm, times the learned scale and hidden^-0.5, linear.

    Returns float64 values of the fp32-rounded logits (the softmax input).
    ``logit_bias`` (the skewed workload's per-expert bias) is added to them.
    """
    x = _f64(x)
    H = x.shape[-1]
    v = rms_normalise(x, eps) * _f64(router_scale)[None, :] * (1.0 / math.sqrt(H))
    logits = v @ _f64(router_w).T
    if logit_bias is not None:
        logits = logits + _f64(logit_bias)[None, :]
    return logits.astype(np.float32).astype(np.float64)


def route(x, router_scale, router_w, per_expert_scale, top_k, eps, logit_bias=None):
    """Full router. Returns a dict with

    ``logits`` [T,E] (fp32 values), ``probs`` [T,E] (softmax over all experts),
    ``topk_idx`` [T,K] int32 (descending logit, ties -> lower index),
    ``renorm`` [T,K] (selected probabilities renormalised to sum 1),
    ``topk_w`` [T,K] (``renorm`` times the per-expert scale),
    ``boundary_tie`` [T] (k-th and (k+1)-th logits closer than NEAR_TIE),
    ``order_tie`` [T] (two selected logits closer than NEAR_TIE).
    """
    logits = router_logits(x, router_scale, router_w, eps, logit_bias)
    T, E = logits.shape
    K = int(top_k)
    # softmax over all experts
    m = logits.max(axis=1, keepdims=True)
    ex = np.exp(logits - m)
    probs = ex / ex.sum(axis=1, keepdims=True)
    # selection: a stable sort of the negated logits keeps equal logits in
    # ascending expert order, i.e. ties go to the lower index
    order = np.argsort(-logits, axis=1, kind="stable")
    idx = order[:, :K]
    sel_p = np.take_along_axis(probs, idx, axis=1)
    renorm = sel_p / sel_p.sum(axis=1, keepdims=True)
    pes = _f64(per_expert_scale)
    topk_w = renorm * pes[idx]
    sorted_l = np.take_along_axis(logits, order, axis=1)
    if K < E:
        boundary = (sorted_l[:, K - 1] - sorted_l[:, K]) < NEAR_TIE
    else:
        boundary = np.zeros(T, dtype=bool)
    if K > 1:
        order_tie = (np.diff(-sorted_l[:, :K], axis=1) < NEAR_TIE).any(axis=1)
    else:
        order_tie = np.zeros(T, dtype=bool)
    return {
        "logits": logits, "probs": probs, "topk_idx": idx.astype(np.int32),
        "renorm": renorm, "topk_w": topk_w,
        "boundary_tie": boundary, "order_tie": order_tie,
    }


# --------------------------------------------------------------------------
# gathered dispatch: group the (token, slot) pairs by expert. [TT]
# "Configurable knobs" (GEMMA4_PREFILL_GATHERED) computes only the routed
# pairs; the pages do not fix an order, the reading here is ascending expert,
# then ascending token (a stable counting sort).
# --------------------------------------------------------------------------
def permute_pairs(topk_idx, num_experts):
    """Returns counts [E], offsets [E+1], perm_token [T*K], perm_slot [T*K],
    inv_row [T*K] (row of pair (t,k) in the grouped order, indexed t*K+k)."""
    idx = np.asarray(topk_idx, dtype=np.int64)
    T, K = idx.shape
    e = idx.reshape(-1)
    t = np.repeat(np.arange(T), K)
    k = np.tile(np.arange(K), T)
    order = np.lexsort((t, e))            # primary key expert, then token
    counts = np.bincount(e, minlength=num_experts).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    inv = np.empty(T * K, dtype=np.int32)
    inv[order] = np.arange(T * K, dtype=np.int32)
    return {
        "counts": counts, "offsets": offsets,
        "perm_token": t[order].astype(np.int32), "perm_slot": k[order].astype(np.int32),
        "inv_row": inv,
    }


# --------------------------------------------------------------------------
# experts and dense MLP: GeGLU with gelu_tanh, [INF2] "How it works (the
# recipe)" (gate_up and down linears), [ONNX] row "Mixture of Experts".
# --------------------------------------------------------------------------
def expert_ffn(x_rows, gate_up, down):
    """down @ (gelu_tanh(gate @ x) * (up @ x)) for rows x [n, H].

    ``gate_up`` [2I, H]: rows [0, I) gate, rows [I, 2I) up; ``down`` [H, I].
    """
    x = _f64(x_rows)
    gu = _f64(gate_up)
    I = gu.shape[0] // 2
    g = x @ gu[:I].T
    u = x @ gu[I:].T
    h = gelu_tanh(g) * u
    return h @ _f64(down).T


def dense_mlp(x, dense_gate_up, dense_down):
    """The shared dense MLP ([ONNX] row "MoE topology"), same GeGLU form."""
    return expert_ffn(x, dense_gate_up, dense_down)


def _expert_weights(weights, e, dtype):
    if dtype == "int8":
        gu = dequantize_int8(weights["expert_gate_up_q"][e], weights["expert_gate_up_scale"][e])
        dn = dequantize_int8(weights["expert_down_q"][e], weights["expert_down_scale"][e])
        return gu, dn
    return weights["expert_gate_up"][e], weights["expert_down"][e]


def _expert(weights, e, dtype):
    """Expert e as a function of its input rows, in the given weight format."""
    if dtype == "fp8":
        return lambda rows: expert_ffn_fp8(rows, weights["expert_gate_up_f8"][e],
                                           weights["expert_gate_up_f8_scale"][e],
                                           weights["expert_down_f8"][e], weights["expert_down_f8_scale"][e])
    gu, dn = _expert_weights(weights, e, dtype)
    return lambda rows: expert_ffn(rows, gu, dn)


def moe_part(x, weights, top_k, eps, expert_dtype="bf16", routing=None):
    """moe = sum_k w[t,k] * expert_{e[t,k]}(x_t), added in k order (the sparse
    top-k form of the MoE branch). Returns ``(moe [T,H] float64, routing)``;
    arguments as for ``moe_block``."""
    x64 = _f64(x)
    if routing is None:
        routing = route(x64, weights["router_scale"], weights["router_w"],
                        weights["per_expert_scale"], top_k, eps, weights.get("logit_bias"))
    idx, w = routing["topk_idx"], routing["topk_w"]
    T, K = idx.shape
    contrib = np.zeros((T, K, x64.shape[1]))
    for e in np.unique(idx):
        tk = np.argwhere(idx == e)                 # (token, slot) pairs routed to e
        out = _expert(weights, int(e), expert_dtype)(x64[tk[:, 0]])
        contrib[tk[:, 0], tk[:, 1]] = w[tk[:, 0], tk[:, 1]][:, None] * out
    moe = np.zeros_like(x64)
    for k in range(K):                             # k order
        moe += contrib[:, k]
    return moe, routing


def moe_block(x, weights, top_k, eps, expert_dtype="bf16", routing=None):
    """y = dense(x) + sum_k w[t,k] * expert_{e[t,k]}(x_t)  (the sparse top-k form).

    ``weights`` uses the keys of ``moe_synth.make_weights``; for
    ``expert_dtype="int8"`` it must also hold ``expert_gate_up_q``,
    ``expert_gate_up_scale``, ``expert_down_q``, ``expert_down_scale``
    (see ``quantize_int8``); for ``"fp8"`` ``expert_gate_up_f8``,
    ``expert_gate_up_f8_scale``, ``expert_down_f8``, ``expert_down_f8_scale``
    (see ``quantize_fp8``). ``routing`` may supply a precomputed ``route``
    result (or one with a different but equally valid index set).
    Returns ``(y [T,H] float64, routing)``.
    """
    x64 = _f64(x)
    moe, routing = moe_part(x64, weights, top_k, eps, expert_dtype, routing)
    dense = dense_mlp(x64, weights["dense_gate_up"], weights["dense_down"])
    return moe + dense, routing


# --------------------------------------------------------------------------
# the layer's FFN around the block: [INF2] "The architecture (a dual-path
# FFN)" (the two branches pass through four feed-forward layernorms) and
# [ONNX] "Truthful graph contracts", row "MoE topology" (post_ff_norm of
# dense + moe, then the residual)
# --------------------------------------------------------------------------
#: the norm positions of ``ffn_layer``: the dense and MoE branches' inputs and
#: outputs, and their sum
FFN_NORMS = ("pre_dense", "pre_moe", "post_dense", "post_moe", "post")


def round_bf16(v):
    """The nearest bfloat16 values, through float32 (ties to even at both
    steps: the kernel forms the value in fp32 and rounds it once to bf16)."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def rms_norm_scaled(v, scale, eps):
    """RMSNorm with a learned per-channel gain, ``v / sqrt(mean(v^2) + eps) *
    scale`` per token; ``scale`` None leaves ``v`` unchanged (no norm there)."""
    if scale is None:
        return _f64(v)
    return rms_normalise(v, eps) * _f64(scale)[None, :]


def ffn_layer(h, weights, norms, top_k, eps, expert_dtype="bf16", routing=None):
    """out = h + N_post(N_post_dense(dense(x_d)) + N_post_moe(moe(x_m))), with
    x_d = N_pre_dense(h) and x_m = N_pre_moe(h) rounded to bf16 (the block's
    input precision); N_k is ``rms_norm_scaled`` with ``norms[k]`` (None: no
    norm at that position) and ``norms["eps"]``. ``eps`` is the router's.

    The router reads the residual stream h itself, not x_m: its own first step
    is a scale-free RMSNorm ([ONNX] row "Router"), the step a router needs
    when its input has not been normalised; the experts read x_m.
    Returns ``(out [T,H] float64, routing)``; routing is that of h.
    """
    h64 = _f64(h)
    ne = norms["eps"]
    xd = h64 if norms["pre_dense"] is None else round_bf16(rms_norm_scaled(h64, norms["pre_dense"], ne))
    xm = h64 if norms["pre_moe"] is None else round_bf16(rms_norm_scaled(h64, norms["pre_moe"], ne))
    dense = dense_mlp(xd, weights["dense_gate_up"], weights["dense_down"])
    if routing is None:
        routing = route(h64, weights["router_scale"], weights["router_w"], weights["per_expert_scale"], top_k,
                        eps, weights.get("logit_bias"))
    moe, routing = moe_part(xm, weights, top_k, eps, expert_dtype, routing)
    s = rms_norm_scaled(dense, norms["post_dense"], ne) + rms_norm_scaled(moe, norms["post_moe"], ne)
    return h64 + rms_norm_scaled(s, norms["post"], ne), routing


def masked_dense_block(x, weights, top_k, eps, expert_dtype="bf16", routing=None):
    """The all-experts-dense form: every expert runs on every token, weighted by
    its router weight, 0 for the unselected ones ([INF2] "How it works (the
    recipe)"; [TT] "Configurable knobs", the legacy all-ones prefill)."""
    x64 = _f64(x)
    if routing is None:
        routing = route(x64, weights["router_scale"], weights["router_w"],
                        weights["per_expert_scale"], top_k, eps, weights.get("logit_bias"))
    idx, w = routing["topk_idx"], routing["topk_w"]
    T = x64.shape[0]
    E = np.asarray(weights["router_w"]).shape[0]
    mask = np.zeros((T, E))
    np.put_along_axis(mask, idx.astype(np.int64), w, axis=1)   # scatter the top-k weights
    y = dense_mlp(x64, weights["dense_gate_up"], weights["dense_down"])
    for e in range(E):
        y = y + mask[:, e:e + 1] * _expert(weights, e, expert_dtype)(x64)
    return y, routing


# --------------------------------------------------------------------------
# int8 experts: [INT8] intro ("per-channel symmetric int8") and "How it
# works" (quantised once, when the checkpoint is loaded). One scale per output
# channel (row): scale = max|w| / 127; q = round-half-even(w / scale), clamped
# to [-127, 127]; a zero row gets scale 0 and q 0. fp32 arithmetic.
# --------------------------------------------------------------------------
def quantize_int8(w_bits):
    """Per-row symmetric int8 of a [..., rows, cols] bf16 tensor -> (q int8, scale fp32)."""
    w = np.asarray(w_bits)
    w32 = (bf16_to_f64(w).astype(np.float32) if w.dtype == np.uint16
           else w.astype(np.float32))
    amax = np.max(np.abs(w32), axis=-1, keepdims=True)
    scale = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    q = np.rint((w32 / safe).astype(np.float32))
    q = np.clip(q, -127, 127)
    q = np.where(scale > 0, q, 0).astype(np.int8)
    return q, scale[..., 0].astype(np.float32)


def dequantize_int8(q, scale):
    return np.asarray(q, dtype=np.float64) * np.asarray(scale, dtype=np.float64)[..., None]


# --------------------------------------------------------------------------
# brute force: the same definition with explicit Python loops and no BLAS,
# for a handful of tokens of the small workload.
# --------------------------------------------------------------------------
# --------------------------------------------------------------------------
# fp8 experts: the vLLM recipe page ("Gemma 4 26B-A4B IT"), ``variants`` ›
# fp8 -- E4M3 expert weights, activations quantised per token at run time.
# E4M3 (OCP, no infinities): sign, 4 exponent bits with bias 7, 3 mantissa
# bits; exponent field 0 holds the subnormals m * 2^-9; S.1111.111 is NaN, so
# the largest finite value is 1.75 * 2^8 = 448.
# --------------------------------------------------------------------------
FP8_MAX = 448.0


def fp8_e4m3_encode(v):
    """float32 values -> E4M3 codes (uint8): the nearest representable value,
    ties to the even code; magnitudes past 448 saturate to 448."""
    a64 = np.asarray(v, dtype=np.float32).astype(np.float64)      # exact
    sign = np.signbit(a64).astype(np.int64) << 7
    a = np.abs(a64)
    code = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # below the smallest normal: multiples of 2^-9 (code 8 is 2^-6 itself)
    code[sub] = np.rint(a[sub] * 512.0).astype(np.int64)          # rint: half to even
    m, ex = np.frexp(a[~sub])                                      # a = m 2^ex, m in [0.5, 1)
    e = ex.astype(np.int64) - 1
    mant = np.rint((2.0 * m - 1.0) * 8.0).astype(np.int64)        # exact operands
    e = np.where(mant == 8, e + 1, e)
    mant = np.where(mant == 8, 0, mant)
    code[~sub] = np.minimum(((e + 7) << 3) | mant, 0x7E)           # saturate at 448
    return (code | sign).astype(np.uint8)


def fp8_e4m3_decode(codes):
    """E4M3 codes -> float64 values (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    e, m = (c >> 3) & 0xF, c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return np.where(c & 0x80, -mag, mag)


def quantize_fp8(v):
    """Per-row E4M3 quantisation of a [..., rows, cols] tensor (bf16 bits or
    floats): scale = max|v| / 448 in fp32, code = encode(v / scale) with the
    division in fp32; an all-zero row gets scale 0 and codes 0. Serves the
    weights (rows = output channels) and the activations (rows = tokens)."""
    a = np.asarray(v)
    v32 = bf16_to_f64(a).astype(np.float32) if a.dtype == np.uint16 else a.astype(np.float32)
    amax = np.max(np.abs(v32), axis=-1, keepdims=True)
    scale = (amax / np.float32(FP8_MAX)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    q = fp8_e4m3_encode((v32 / safe).astype(np.float32))
    q = np.where(scale > 0, q, 0).astype(np.uint8)
    return q, scale[..., 0].astype(np.float32)


def dequantize_fp8(q, scale):
    return fp8_e4m3_decode(q) * np.asarray(scale, dtype=np.float64)[..., None]


def expert_ffn_fp8(x_rows, gu_q, gu_scale, dn_q, dn_scale):
    """An fp8 expert on input rows x [n, H] (bf16 values): each row quantised
    per token, the GeGLU on the dequantised rows and weights, h rounded to bf16
    and quantised per row, then the down projection.

    Reading (the recipe page fixes only "dynamic per-token activation
    quantization"): an activation is quantised from the tensor the model holds
    between its operators, which in a bf16 model is a bf16 tensor. x arrives in
    bf16; h, the GeGLU's output and the down projection's input, is such a
    tensor too, so it is rounded to bf16 before its per-row quantisation. (On
    the bf16 path nothing is quantised and the oracle keeps h exact.)"""
    x32 = _f64(x_rows).astype(np.float32)                          # bf16 values: exact
    xq = dequantize_fp8(*quantize_fp8(x32))
    gu = dequantize_fp8(gu_q, gu_scale)
    I = gu.shape[0] // 2
    h = round_bf16(gelu_tanh(xq @ gu[:I].T) * (xq @ gu[I:].T))
    hq = dequantize_fp8(*quantize_fp8(h.astype(np.float32)))       # bf16 values: exact
    return hq @ dequantize_fp8(dn_q, dn_scale).T


def brute_force_block(x, weights, top_k, eps, tokens):
    """y for the listed token indices, computed element by element in float64."""
    X = _f64(x)
    s = _f64(weights["router_scale"])
    Wr = _f64(weights["router_w"])
    pes = _f64(weights["per_expert_scale"])
    bias = weights.get("logit_bias")
    bias = None if bias is None else _f64(bias)
    E, H = Wr.shape
    out = []
    for t in tokens:
        xt = [float(v) for v in X[t]]
        ms = math.fsum(v * v for v in xt) / H
        inv = 1.0 / math.sqrt(ms + eps)
        v = [xt[h] * inv * float(s[h]) / math.sqrt(H) for h in range(H)]
        logit = []
        for e in range(E):
            le = math.fsum(v[h] * float(Wr[e, h]) for h in range(H))
            if bias is not None:
                le += float(bias[e])
            logit.append(float(np.float32(le)))
        chosen = []
        for _ in range(top_k):
            best = None
            for e in range(E):
                if e in chosen:
                    continue
                if best is None or logit[e] > logit[best]:
                    best = e
            chosen.append(best)
        mx = max(logit)
        z = math.fsum(math.exp(l - mx) for l in logit)
        p = [math.exp(logit[e] - mx) / z for e in chosen]
        ps = math.fsum(p)
        wts = [p[i] / ps * float(pes[chosen[i]]) for i in range(top_k)]
        y = [0.0] * H

        def ffn(gu, dn):
            gu = _f64(gu)
            dn = _f64(dn)
            inter = gu.shape[0] // 2
            hvec = []
            for j in range(inter):
                g = math.fsum(float(gu[j, i]) * xt[i] for i in range(H))
                u = math.fsum(float(gu[inter + j, i]) * xt[i] for i in range(H))
                gl = 0.5 * g * (1.0 + math.tanh(math.sqrt(2.0 / math.pi) * (g + 0.044715 * g ** 3)))
                hvec.append(gl * u)
            return [math.fsum(float(dn[i, j]) * hvec[j] for j in range(inter)) for i in range(H)]

        for k, e in enumerate(chosen):
            o = ffn(weights["expert_gate_up"][e], weights["expert_down"][e])
            for i in range(H):
                y[i] += wts[k] * o[i]
        d = ffn(weights["dense_gate_up"], weights["dense_down"])
        out.append([y[i] + d[i] for i in range(H)])
    return np.array(out)
