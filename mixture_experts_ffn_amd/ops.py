"""Python binding of libmoe_ffn.so: the entry points of include/moe.h with the
same names, taking torch tensors for device memory and the current HIP stream.

Argument marshalling only: every step of the block runs in the HIP kernels of
the library. There is no CPU or PyTorch fallback; a missing library or a bad
argument raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
from typing import Optional

import torch

from . import _abi
from ._abi import MoeDebug, MoeDims, MoeWeights


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where}: {_abi.STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


@dataclasses.dataclass
class BlockDims:
    hidden: int
    num_experts: int
    top_k: int
    expert_inter: int
    dense_inter: int
    rms_eps: float = 1e-6

    def c(self) -> MoeDims:
        return MoeDims(self.hidden, self.num_experts, self.top_k, self.expert_inter,
                       self.dense_inter, self.rms_eps)


@dataclasses.dataclass
class LayerWeights:
    """Device tensors of one layer (layouts as in include/moe.h). The expert and
    dense matrices must be in the tiled layout for moe_block: tile_layer()
    returns such a copy of a layer held row-major."""
    router_scale: torch.Tensor            # [H] bf16
    router_w: torch.Tensor                # [E, H] bf16
    per_expert_scale: torch.Tensor        # [E] fp32
    expert_gate_up: torch.Tensor          # [E, 2I, H] bf16, int8, or E4M3 codes (float8_e4m3fn or uint8)
    expert_down: torch.Tensor             # [E, H, I] same format
    dense_gate_up: torch.Tensor           # [2Id, H] bf16
    dense_down: torch.Tensor              # [H, Id] bf16
    logit_bias: Optional[torch.Tensor] = None   # [E] fp32
    gate_up_scale: Optional[torch.Tensor] = None  # [E, 2I] fp32 (int8, E4M3)
    down_scale: Optional[torch.Tensor] = None     # [E, H] fp32 (int8, E4M3)
    layout: int = _abi.MOE_LAYOUT_ROWS            # of the four expert / dense matrices

    @property
    def expert_dtype(self) -> int:
        return _weight_format(self.expert_gate_up.dtype)

    def check(self, dims: "BlockDims"):
        """Every tensor's shape and dtype against dims, and one device for all."""
        H, E, I, Id = dims.hidden, dims.num_experts, dims.expert_inter, dims.dense_inter
        bf, f32 = (torch.bfloat16,), (torch.float32,)
        _want(self.router_scale, "router_scale", (H,), bf)
        _want(self.router_w, "router_w", (E, H), bf)
        _want(self.per_expert_scale, "per_expert_scale", (E,), f32)
        if self.logit_bias is not None:
            _want(self.logit_bias, "logit_bias", (E,), f32)
        fmt = (torch.bfloat16, torch.int8) + _ONE_BYTE
        _want(self.expert_gate_up, "expert_gate_up", (E, 2 * I, H), fmt)
        dn_fmt = (torch.uint8, torch.float8_e4m3fn) if self.expert_gate_up.dtype in (torch.uint8,
                                                                                    torch.float8_e4m3fn) \
            else (self.expert_gate_up.dtype,)
        _want(self.expert_down, "expert_down", (E, H, I), dn_fmt)
        if self.expert_gate_up.dtype != torch.bfloat16:
            if self.gate_up_scale is None or self.down_scale is None:
                raise ValueError("1-byte expert weights need gate_up_scale and down_scale")
            _want(self.gate_up_scale, "gate_up_scale", (E, 2 * I), f32)
            _want(self.down_scale, "down_scale", (E, H), f32)
        _want(self.dense_gate_up, "dense_gate_up", (2 * Id, H), bf)
        _want(self.dense_down, "dense_down", (H, Id), bf)
        _same_device(*[(k, v) for k, v in vars(self).items() if isinstance(v, torch.Tensor)])
        return self

    def c(self) -> MoeWeights:
        def ptr(t):
            return None if t is None else _dev(t, "weight").data_ptr()
        return MoeWeights(ptr(self.router_scale), ptr(self.router_w), ptr(self.per_expert_scale),
                          ptr(self.logit_bias), ptr(self.expert_gate_up), ptr(self.expert_down),
                          self.expert_dtype, ptr(self.gate_up_scale), ptr(self.down_scale),
                          ptr(self.dense_gate_up), ptr(self.dense_down), int(self.layout))


def _lib():
    return _abi.load_library()


def _dev(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


_ONE_BYTE = (torch.int8, torch.uint8, torch.float8_e4m3fn)


def _want(t, name: str, shape, dtypes) -> torch.Tensor:
    """Shape and dtype of an argument against what the dims imply (checked
    before the device, so that a mismatch raises wherever the tensor lives)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {list(dtypes)}")
    return t


def _tokens(x, name: str, hidden: int) -> int:
    """T of an activation [T, hidden] bf16."""
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if x.dim() != 2 or x.shape[1] != hidden:
        raise ValueError(f"{name} has shape {tuple(x.shape)}, expected (T, {hidden})")
    _want(x, name, x.shape, (torch.bfloat16,))
    return int(x.shape[0])


def _same_device(*named):
    devs = {t.device for _, t in named if t is not None}
    if len(devs) > 1:
        raise ValueError("arguments live on different devices: "
                         + ", ".join(f"{n} on {t.device}" for n, t in named if t is not None))


def _debug_outputs(debug, dims: "BlockDims", T: int):
    """The device outputs a debug struct made by new_debug() names must hold
    what the block writes into them."""
    outs = getattr(debug, "_outputs", None) if debug is not None else None
    if not outs:
        return []
    K, E = dims.top_k, dims.num_experts
    need = {"topk_idx": (T * K, torch.int32), "topk_w": (T * K, torch.float32), "counts": (E, torch.int32),
            "offsets": (E + 1, torch.int32), "perm_token": (T * K, torch.int32), "inv_row": (T * K, torch.int32)}
    for k, t in outs.items():
        n, dt = need[k]
        if t.dtype != dt or t.numel() < n:
            raise ValueError(f"debug output {k} must hold at least {n} {dt} values (has {t.numel()} {t.dtype})")
    return list(outs.items())


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(rc: int, where: str):
    if rc != _abi.MOE_OK:
        raise MoEError(rc, where, _lib().moe_last_error().decode())


def moe_workspace_bytes(dims: BlockDims, T: int) -> int:
    n = _lib().moe_workspace_bytes(ctypes.byref(dims.c()), int(T))
    if n == 0:
        raise MoEError(_abi.MOE_ERR_SHAPE, "moe_workspace_bytes", _lib().moe_last_error().decode())
    return int(n)


def _workspace(dims, T, device, workspace):
    need = moe_workspace_bytes(dims, T)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    return _dev(workspace, "workspace"), need


def moe_route(dims: BlockDims, weights: LayerWeights, x: torch.Tensor, topk_idx=None,
              topk_w=None, workspace=None, stream=None):
    """Router alone: returns (topk_idx [T,K] int32, topk_w [T,K] fp32)."""
    T = _tokens(x, "x", dims.hidden)
    weights.check(dims)
    if topk_idx is not None:
        _want(topk_idx, "topk_idx", (T, dims.top_k), (torch.int32,))
    if topk_w is not None:
        _want(topk_w, "topk_w", (T, dims.top_k), (torch.float32,))
    _same_device(("x", x), ("router_w", weights.router_w), ("topk_idx", topk_idx), ("topk_w", topk_w))
    x = _dev(x, "x")
    if topk_idx is None:
        topk_idx = torch.empty((T, dims.top_k), dtype=torch.int32, device=x.device)
    if topk_w is None:
        topk_w = torch.empty((T, dims.top_k), dtype=torch.float32, device=x.device)
    ws, _ = _workspace(dims, T, x.device, workspace)
    rc = _lib().moe_route(ctypes.byref(dims.c()), ctypes.byref(weights.c()), x.data_ptr(), T,
                          _dev(topk_idx, "topk_idx").data_ptr(), _dev(topk_w, "topk_w").data_ptr(),
                          ws.data_ptr(), ws.numel(), _stream(stream))
    _check(rc, "moe_route")
    return topk_idx, topk_w


def moe_block(dims: BlockDims, weights: LayerWeights, x: torch.Tensor, y=None,
              debug: Optional[MoeDebug] = None, workspace=None, stream=None) -> torch.Tensor:
    """The whole block: y = dense(x) + sum_k w_k expert_k(x) (bf16 [T, H])."""
    T = _tokens(x, "x", dims.hidden)
    weights.check(dims)
    if y is not None:
        _want(y, "y", (T, dims.hidden), (torch.bfloat16,))
    _same_device(("x", x), ("router_w", weights.router_w), ("y", y), *_debug_outputs(debug, dims, T))
    x = _dev(x, "x")
    if y is None:
        y = torch.empty((T, dims.hidden), dtype=torch.bfloat16, device=x.device)
    ws, _ = _workspace(dims, T, x.device, workspace)
    rc = _lib().moe_block(ctypes.byref(dims.c()), ctypes.byref(weights.c()), x.data_ptr(), T,
                          _dev(y, "y").data_ptr(), ctypes.byref(debug) if debug is not None else None,
                          ws.data_ptr(), ws.numel(), _stream(stream))
    _check(rc, "moe_block")
    return y


def moe_block_noalloc(dims: BlockDims, weights: LayerWeights, x: torch.Tensor, y: torch.Tensor,
                      debug: Optional[MoeDebug] = None, stream=None) -> torch.Tensor:
    """moe_block on the library's own scratch array: no workspace, nothing
    allocated (y must be given). Calls that overlap on one device race."""
    T = _tokens(x, "x", dims.hidden)
    weights.check(dims)
    _want(y, "y", (T, dims.hidden), (torch.bfloat16,))
    _same_device(("x", x), ("router_w", weights.router_w), ("y", y), *_debug_outputs(debug, dims, T))
    rc = _lib().moe_block_noalloc(ctypes.byref(dims.c()), ctypes.byref(weights.c()), _dev(x, "x").data_ptr(), T,
                                  _dev(y, "y").data_ptr(), ctypes.byref(debug) if debug is not None else None,
                                  _stream(stream))
    _check(rc, "moe_block_noalloc")
    return y


def dense_mlp(dims: BlockDims, dense_gate_up: torch.Tensor, dense_down: torch.Tensor,
              x: torch.Tensor, y=None, workspace=None, stream=None) -> torch.Tensor:
    """The shared dense MLP alone (bf16 [T, H])."""
    T = _tokens(x, "x", dims.hidden)
    _want(dense_gate_up, "dense_gate_up", (2 * dims.dense_inter, dims.hidden), (torch.bfloat16,))
    _want(dense_down, "dense_down", (dims.hidden, dims.dense_inter), (torch.bfloat16,))
    if y is not None:
        _want(y, "y", (T, dims.hidden), (torch.bfloat16,))
    _same_device(("x", x), ("dense_gate_up", dense_gate_up), ("dense_down", dense_down), ("y", y))
    x = _dev(x, "x")
    if y is None:
        y = torch.empty((T, dims.hidden), dtype=torch.bfloat16, device=x.device)
    ws, _ = _workspace(dims, T, x.device, workspace)
    rc = _lib().dense_mlp(ctypes.byref(dims.c()), _dev(dense_gate_up, "dense_gate_up").data_ptr(),
                          _dev(dense_down, "dense_down").data_ptr(), x.data_ptr(), T,
                          _dev(y, "y").data_ptr(), ws.data_ptr(), ws.numel(), _stream(stream))
    _check(rc, "dense_mlp")
    return y


@dataclasses.dataclass
class FfnNorms:
    """Gains of the layer's feed-forward norms around the block (bf16 [H]
    device tensors, or None: no norm at that position); see moe_ffn_layer."""
    pre_dense: Optional[torch.Tensor] = None
    pre_moe: Optional[torch.Tensor] = None
    post_dense: Optional[torch.Tensor] = None
    post_moe: Optional[torch.Tensor] = None
    post: Optional[torch.Tensor] = None
    eps: float = 1e-6

    def check(self, dims: "BlockDims"):
        for k in ("pre_dense", "pre_moe", "post_dense", "post_moe", "post"):
            if getattr(self, k) is not None:
                _want(getattr(self, k), k, (dims.hidden,), (torch.bfloat16,))
        return self

    def tensors(self):
        return [(k, getattr(self, k)) for k in ("pre_dense", "pre_moe", "post_dense", "post_moe", "post")]

    def c(self) -> _abi.MoeFfnNorms:
        def p(t, name):
            return None if t is None else _dev(t, name).data_ptr()
        return _abi.MoeFfnNorms(p(self.pre_dense, "pre_dense"), p(self.pre_moe, "pre_moe"),
                                p(self.post_dense, "post_dense"), p(self.post_moe, "post_moe"),
                                p(self.post, "post"), self.eps)


def moe_ffn_workspace_bytes(dims: BlockDims, T: int) -> int:
    n = _lib().moe_ffn_workspace_bytes(ctypes.byref(dims.c()), T)
    if n == 0:
        raise MoEError(_abi.MOE_ERR_SHAPE, "moe_ffn_workspace_bytes", _lib().moe_last_error().decode())
    return n


def moe_ffn_layer(dims: BlockDims, weights: LayerWeights, norms: Optional[FfnNorms], h: torch.Tensor,
                  out=None, debug: Optional[MoeDebug] = None, workspace=None, stream=None) -> torch.Tensor:
    """The layer's FFN: out = h + N_post(N_post_dense(dense(x_d)) + N_post_moe(moe(x_m)))
    with x_d, x_m the pre-normed h and the router on h (bf16 [T, H] in and out)."""
    T = _tokens(h, "h", dims.hidden)
    weights.check(dims)
    if norms is not None:
        norms.check(dims)
    if out is not None:
        _want(out, "out", (T, dims.hidden), (torch.bfloat16,))
    _same_device(("h", h), ("router_w", weights.router_w), ("out", out),
                 *(norms.tensors() if norms is not None else []), *_debug_outputs(debug, dims, T))
    h = _dev(h, "h")
    if out is None:
        out = torch.empty((T, dims.hidden), dtype=torch.bfloat16, device=h.device)
    need = moe_ffn_workspace_bytes(dims, T)
    ws = workspace if workspace is not None else torch.empty(need, dtype=torch.uint8, device=h.device)
    ws = _dev(ws, "workspace")
    cn = norms.c() if norms is not None else None
    rc = _lib().moe_ffn_layer(ctypes.byref(dims.c()), ctypes.byref(weights.c()),
                              ctypes.byref(cn) if cn is not None else None, h.data_ptr(), T,
                              _dev(out, "out").data_ptr(), ctypes.byref(debug) if debug is not None else None,
                              ws.data_ptr(), ws.numel(), _stream(stream))
    _check(rc, "moe_ffn_layer")
    return out


def moe_prefill_chunk_tokens(chunk_tokens: int = 0) -> int:
    """The chunk size the chunked prefill uses for a requested one (0: the default)."""
    return int(_lib().moe_prefill_chunk_tokens(int(chunk_tokens)))


def moe_prefill_workspace_bytes(dims: BlockDims, chunk_tokens: int = 0) -> int:
    n = _lib().moe_prefill_workspace_bytes(ctypes.byref(dims.c()), int(chunk_tokens))
    if n == 0:
        raise MoEError(_abi.MOE_ERR_SHAPE, "moe_prefill_workspace_bytes", _lib().moe_last_error().decode())
    return n


def moe_prefill_chunked(dims: BlockDims, weights: LayerWeights, norms: Optional[FfnNorms], h: torch.Tensor,
                        chunk_tokens: int = 0, out=None, workspace=None, stream=None) -> torch.Tensor:
    """Chunked prefill: consecutive chunks of h through the block (norms None)
    or the layer's FFN (norms given), reusing one chunk's workspace."""
    T = _tokens(h, "h", dims.hidden)
    weights.check(dims)
    if norms is not None:
        norms.check(dims)
    if out is not None:
        _want(out, "out", (T, dims.hidden), (torch.bfloat16,))
    _same_device(("h", h), ("router_w", weights.router_w), ("out", out),
                 *(norms.tensors() if norms is not None else []))
    h = _dev(h, "h")
    if out is None:
        out = torch.empty((T, dims.hidden), dtype=torch.bfloat16, device=h.device)
    if workspace is None:
        workspace = torch.empty(moe_prefill_workspace_bytes(dims, chunk_tokens), dtype=torch.uint8,
                                device=h.device)
    ws = _dev(workspace, "workspace")
    cn = norms.c() if norms is not None else None
    rc = _lib().moe_prefill_chunked(ctypes.byref(dims.c()), ctypes.byref(weights.c()),
                                    ctypes.byref(cn) if cn is not None else None, h.data_ptr(), T,
                                    int(chunk_tokens), _dev(out, "out").data_ptr(), ws.data_ptr(), ws.numel(),
                                    _stream(stream))
    _check(rc, "moe_prefill_chunked")
    return out


def _weight_format(dt) -> int:
    if dt == torch.bfloat16:
        return _abi.MOE_DTYPE_BF16
    if dt == torch.int8:
        return _abi.MOE_DTYPE_INT8
    if dt in (torch.uint8, torch.float8_e4m3fn):
        return _abi.MOE_DTYPE_FP8
    raise TypeError(f"expert weights must be bf16, int8 or E4M3 codes (float8_e4m3fn / uint8), got {dt}")


def moe_quantize_fp8(w: torch.Tensor, q=None, scale=None, stream=None):
    """Per-row E4M3 of a bf16 tensor [..., cols]: returns (codes float8_e4m3fn, scale fp32 [...])."""
    _want(w, "w", w.shape, (torch.bfloat16,))
    if q is not None:
        _want(q, "q", w.shape, (torch.uint8, torch.float8_e4m3fn))
    if scale is not None:
        _want(scale, "scale", w.shape[:-1], (torch.float32,))
    _same_device(("w", w), ("q", q), ("scale", scale))
    w = _dev(w, "w")
    cols = w.shape[-1]
    rows = w.numel() // cols
    if q is None:
        q = torch.empty(w.shape, dtype=torch.float8_e4m3fn, device=w.device)
    if scale is None:
        scale = torch.empty(w.shape[:-1], dtype=torch.float32, device=w.device)
    rc = _lib().moe_quantize_fp8(w.data_ptr(), rows, cols, _dev(q, "q").data_ptr(),
                                 _dev(scale, "scale").data_ptr(), _stream(stream))
    _check(rc, "moe_quantize_fp8")
    return q, scale


def moe_quantize_int8(w: torch.Tensor, q=None, scale=None, stream=None):
    """Per-row symmetric int8 of a bf16 tensor [..., cols]: returns (q int8, scale fp32 [...])."""
    _want(w, "w", w.shape, (torch.bfloat16,))
    if q is not None:
        _want(q, "q", w.shape, (torch.int8,))
    if scale is not None:
        _want(scale, "scale", w.shape[:-1], (torch.float32,))
    _same_device(("w", w), ("q", q), ("scale", scale))
    w = _dev(w, "w")
    cols = w.shape[-1]
    rows = w.numel() // cols
    if q is None:
        q = torch.empty(w.shape, dtype=torch.int8, device=w.device)
    if scale is None:
        scale = torch.empty(w.shape[:-1], dtype=torch.float32, device=w.device)
    rc = _lib().moe_quantize_int8(w.data_ptr(), rows, cols, _dev(q, "q").data_ptr(),
                                  _dev(scale, "scale").data_ptr(), _stream(stream))
    _check(rc, "moe_quantize_int8")
    return q, scale


def moe_tile_weights(w: torch.Tensor, out=None, stream=None) -> torch.Tensor:
    """Tiled-layout copy of a row-major bf16 or int8 matrix [..., rows, cols]
    (all leading dimensions stacked as rows). Same shape and dtype; the data is
    re-laid into 16 x 64 tiles (include/moe.h, MOE_LAYOUT_TILED)."""
    dtype = _weight_format(w.dtype)
    if out is not None:
        _want(out, "out", w.shape, (w.dtype,))
    _same_device(("w", w), ("out", out))
    w = _dev(w, "w")
    cols = w.shape[-1]
    rows = w.numel() // cols
    if out is None:
        out = torch.empty_like(w)
    rc = _lib().moe_tile_weights(w.data_ptr(), rows, cols, dtype, _dev(out, "out").data_ptr(),
                                 _stream(stream))
    _check(rc, "moe_tile_weights")
    return out


def tile_layer(w: LayerWeights, stream=None) -> LayerWeights:
    """A copy of a row-major layer with its expert and dense matrices tiled."""
    if w.layout == _abi.MOE_LAYOUT_TILED:
        return w
    return dataclasses.replace(
        w, expert_gate_up=moe_tile_weights(w.expert_gate_up, stream=stream),
        expert_down=moe_tile_weights(w.expert_down, stream=stream),
        dense_gate_up=moe_tile_weights(w.dense_gate_up, stream=stream),
        dense_down=moe_tile_weights(w.dense_down, stream=stream), layout=_abi.MOE_LAYOUT_TILED)


class BlockCall:
    """moe_block with its arguments marshalled once, for repeated calls on the
    same tensors (the ctypes structures are built here, not per call)."""

    def __init__(self, dims: BlockDims, weights: LayerWeights, x: torch.Tensor, y=None,
                 workspace=None):
        T = _tokens(x, "x", dims.hidden)
        weights.check(dims)
        if y is not None:
            _want(y, "y", (T, dims.hidden), (torch.bfloat16,))
        _same_device(("x", x), ("router_w", weights.router_w), ("y", y))
        self.dims = dims
        self.x = _dev(x, "x")
        self.T = x.shape[0]
        self.y = y if y is not None else torch.empty((self.T, dims.hidden), dtype=torch.bfloat16,
                                                     device=x.device)
        self.ws, _ = _workspace(dims, self.T, x.device, workspace)
        self.weights = weights          # keeps the tensors alive
        self._dims = dims.c()
        self._w = weights.c()

    def __call__(self, debug: Optional[MoeDebug] = None, stream=None) -> torch.Tensor:
        _same_device(("x", self.x), *_debug_outputs(debug, self.dims, self.T))
        rc = _lib().moe_block(ctypes.byref(self._dims), ctypes.byref(self._w), self.x.data_ptr(),
                              self.T, self.y.data_ptr(),
                              ctypes.byref(debug) if debug is not None else None,
                              self.ws.data_ptr(), self.ws.numel(), _stream(stream))
        _check(rc, "moe_block")
        return self.y


class FfnCall:
    """moe_ffn_layer with its arguments marshalled once, for repeated calls on
    the same tensors."""

    def __init__(self, dims: BlockDims, weights: LayerWeights, norms: Optional[FfnNorms], h: torch.Tensor,
                 out=None, workspace=None):
        T = _tokens(h, "h", dims.hidden)
        weights.check(dims)
        if norms is not None:
            norms.check(dims)
        if out is not None:
            _want(out, "out", (T, dims.hidden), (torch.bfloat16,))
        _same_device(("h", h), ("router_w", weights.router_w), ("out", out),
                     *(norms.tensors() if norms is not None else []))
        self.dims = dims
        self.h = _dev(h, "h")
        self.T = h.shape[0]
        self.out = out if out is not None else torch.empty((self.T, dims.hidden), dtype=torch.bfloat16,
                                                           device=h.device)
        need = moe_ffn_workspace_bytes(dims, self.T)
        self.ws = _dev(workspace if workspace is not None
                       else torch.empty(need, dtype=torch.uint8, device=h.device), "workspace")
        self.weights, self.norms = weights, norms  # keep the tensors alive
        self._dims = dims.c()
        self._w = weights.c()
        self._n = norms.c() if norms is not None else None

    def __call__(self, debug: Optional[MoeDebug] = None, stream=None) -> torch.Tensor:
        _same_device(("h", self.h), *_debug_outputs(debug, self.dims, self.T))
        rc = _lib().moe_ffn_layer(ctypes.byref(self._dims), ctypes.byref(self._w),
                                  ctypes.byref(self._n) if self._n is not None else None, self.h.data_ptr(),
                                  self.T, self.out.data_ptr(), ctypes.byref(debug) if debug is not None else None,
                                  self.ws.data_ptr(), self.ws.numel(), _stream(stream))
        _check(rc, "moe_ffn_layer")
        return self.out


def new_debug(path: int = _abi.MOE_PATH_AUTO, **outputs) -> MoeDebug:
    """A moe_debug struct; keyword arguments name device tensors for its outputs."""
    d = MoeDebug()
    d.path = path
    allowed = ("topk_idx", "topk_w", "counts", "offsets", "perm_token", "inv_row")
    for k, t in outputs.items():
        if k not in allowed:
            raise ValueError(f"unknown debug output {k} (one of {allowed})")
        setattr(d, k, _dev(t, k).data_ptr())
    d._outputs = dict(outputs)  # sizes are checked against T at each call
    return d
