"""The C-ABI library: it loads, exports every declared symbol, sizes its
workspace, and rejects bad arguments before launching anything.

No test here launches a kernel: argument checks run on the host before any
HIP call, so they work without a GPU.
"""
import ctypes
import re

import pytest

from mixture_experts_ffn_amd import _abi



@pytest.fixture(scope="module")
def L():
    return _abi.load_library()


def _declared_functions():
    src = open(_abi.HEADER_PATH).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if not n.startswith("MOE_") and n not in ("if", "defined")))


def test_header_declares_the_boundary():
    assert set(_declared_functions()) == set(_abi.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    for name in _declared_functions():
        assert hasattr(L, name), name


def _real():
    return _abi.MoeDims(2816, 128, 8, 704, 2112, 1e-6)


def test_workspace_bytes(L):
    d = _real()
    n8 = L.moe_workspace_bytes(ctypes.byref(d), 8)
    n2048 = L.moe_workspace_bytes(ctypes.byref(d), 2048)
    assert 0 < n8 < n2048
    assert n8 % 256 == 0 and n2048 % 256 == 0
    # grouped rows [T*K, H] bf16 dominate at large T
    assert n2048 >= 2048 * 8 * 2816 * 2 + 2048 * 8 * 704 * 2
    assert L.moe_workspace_bytes(ctypes.byref(d), 0) > 0
    assert L.moe_workspace_bytes(ctypes.byref(d), -1) == 0
    bad = _abi.MoeDims(2816, 128, 9, 704, 2112, 1e-6)
    assert L.moe_workspace_bytes(ctypes.byref(bad), 8) == 0
    assert b"top_k" in L.moe_last_error()


FAKE = 0x7F0000000000  # 256-aligned host-side value; never dereferenced


def _weights(**over):
    w = _abi.MoeWeights(FAKE, FAKE, FAKE, None, FAKE, FAKE, _abi.MOE_DTYPE_BF16, None, None, FAKE, FAKE,
                        _abi.MOE_LAYOUT_TILED)
    for k, v in over.items():
        setattr(w, k, v)
    return w


@pytest.mark.parametrize("dims,code", [
    ((2816, 128, 8, 704, 2112), 0),
    ((2816, 128, 9, 704, 2112), _abi.MOE_ERR_UNSUPPORTED),
    ((2816, 300, 8, 704, 2112), _abi.MOE_ERR_UNSUPPORTED),
    ((2800, 128, 8, 704, 2112), _abi.MOE_ERR_SHAPE),
    ((2816, 128, 8, 700, 2112), _abi.MOE_ERR_SHAPE),
    ((2816, 128, 8, 704, 2100), _abi.MOE_ERR_SHAPE),
    ((2816, 4, 8, 704, 2112), _abi.MOE_ERR_SHAPE),
    ((2816, 128, 0, 704, 2112), _abi.MOE_ERR_SHAPE),
])
def test_dims_validation(L, dims, code):
    d = _abi.MoeDims(*dims, 1e-6)
    n = L.moe_workspace_bytes(ctypes.byref(d), 16)
    assert (n > 0) == (code == 0)
    if code:
        w = _weights()
        rc = L.moe_block(ctypes.byref(d), ctypes.byref(w), FAKE, 16, FAKE, None, FAKE, 1 << 40, None)
        assert rc == code, L.moe_last_error()


def test_block_argument_errors(L):
    d = _real()
    ws = L.moe_workspace_bytes(ctypes.byref(d), 8)
    ok = dict(x=FAKE, T=8, y=FAKE, ws=FAKE, ws_bytes=ws)

    def call(w=None, **kw):
        a = dict(ok, **kw)
        w = w or _weights()
        return L.moe_block(ctypes.byref(d), ctypes.byref(w), a["x"], a["T"], a["y"], None,
                           a["ws"], a["ws_bytes"], None)

    assert call(x=None) == _abi.MOE_ERR_NULL
    assert call(y=None) == _abi.MOE_ERR_NULL
    assert call(ws=None) == _abi.MOE_ERR_NULL
    assert call(x=FAKE + 8) == _abi.MOE_ERR_ALIGN
    assert call(ws=FAKE + 16) == _abi.MOE_ERR_ALIGN
    assert call(ws_bytes=ws - 1) == _abi.MOE_ERR_WORKSPACE
    assert call(T=-1) == _abi.MOE_ERR_SHAPE
    assert call(T=_abi.MOE_MAX_TOKENS + 1) == _abi.MOE_ERR_SHAPE
    assert call(w=_weights(router_w=None)) == _abi.MOE_ERR_NULL
    assert call(w=_weights(expert_dtype=7)) == _abi.MOE_ERR_UNSUPPORTED
    # int8 experts need their scales
    assert call(w=_weights(expert_dtype=_abi.MOE_DTYPE_INT8)) == _abi.MOE_ERR_NULL
    assert b"gate_up_scale" in L.moe_last_error()
    # the block reads tiled weights only
    assert call(w=_weights(layout=_abi.MOE_LAYOUT_ROWS)) == _abi.MOE_ERR_UNSUPPORTED
    assert b"moe_tile_weights" in L.moe_last_error()
    # an empty batch is a valid no-op (nothing is launched)
    assert call(T=0, ws_bytes=L.moe_workspace_bytes(ctypes.byref(d), 0)) == _abi.MOE_OK
    assert call(T=0, x=None, y=None, ws=None, ws_bytes=0) == _abi.MOE_OK


def test_stream_path_limits(L):
    d = _real()
    T = _abi.MOE_STREAM_MAX_TOKENS + 1
    ws = L.moe_workspace_bytes(ctypes.byref(d), T)
    dbg = _abi.MoeDebug()
    dbg.path = _abi.MOE_PATH_STREAM
    w = _weights()
    rc = L.moe_block(ctypes.byref(d), ctypes.byref(w), FAKE, T, FAKE, ctypes.byref(dbg), FAKE, ws, None)
    assert rc == _abi.MOE_ERR_UNSUPPORTED
    dbg.path = 9
    rc = L.moe_block(ctypes.byref(d), ctypes.byref(w), FAKE, 8, FAKE, ctypes.byref(dbg), FAKE, ws, None)
    assert rc == _abi.MOE_ERR_UNSUPPORTED


def test_route_dense_quant_argument_errors(L):
    d = _real()
    ws = L.moe_workspace_bytes(ctypes.byref(d), 8)
    w = _weights()
    assert L.moe_route(ctypes.byref(d), ctypes.byref(w), FAKE, 8, None, FAKE, FAKE, ws, None) == _abi.MOE_ERR_NULL
    assert L.moe_route(ctypes.byref(d), ctypes.byref(w), FAKE, 8, FAKE, FAKE, FAKE, 16, None) == _abi.MOE_ERR_WORKSPACE
    assert L.dense_mlp(ctypes.byref(d), None, FAKE, FAKE, 8, FAKE, FAKE, ws, None) == _abi.MOE_ERR_NULL
    assert L.dense_mlp(ctypes.byref(d), FAKE, FAKE, FAKE, 0, FAKE, FAKE, ws, None) == _abi.MOE_OK
    assert L.moe_quantize_int8(FAKE, 10, 12, FAKE, FAKE, None) == _abi.MOE_ERR_SHAPE
    assert L.moe_quantize_int8(FAKE, -1, 16, FAKE, FAKE, None) == _abi.MOE_ERR_SHAPE
    assert L.moe_quantize_int8(FAKE, 0, 16, FAKE, FAKE, None) == _abi.MOE_OK
    assert L.moe_quantize_int8(FAKE + 4, 4, 16, FAKE, FAKE, None) == _abi.MOE_ERR_ALIGN


def test_tile_weights_argument_errors(L):
    OTHER = FAKE + 4096
    assert L.moe_tile_weights(FAKE, 24, 128, _abi.MOE_DTYPE_BF16, OTHER, None) == _abi.MOE_ERR_SHAPE
    assert L.moe_tile_weights(FAKE, 32, 96, _abi.MOE_DTYPE_BF16, OTHER, None) == _abi.MOE_ERR_SHAPE
    assert L.moe_tile_weights(FAKE, -16, 128, _abi.MOE_DTYPE_INT8, OTHER, None) == _abi.MOE_ERR_SHAPE
    assert L.moe_tile_weights(FAKE, 32, 128, 5, OTHER, None) == _abi.MOE_ERR_UNSUPPORTED
    assert L.moe_tile_weights(None, 32, 128, _abi.MOE_DTYPE_BF16, OTHER, None) == _abi.MOE_ERR_NULL
    assert L.moe_tile_weights(FAKE + 8, 32, 128, _abi.MOE_DTYPE_BF16, OTHER, None) == _abi.MOE_ERR_ALIGN
    assert L.moe_tile_weights(FAKE, 32, 128, _abi.MOE_DTYPE_BF16, FAKE, None) == _abi.MOE_ERR_SHAPE
    assert L.moe_tile_weights(FAKE, 0, 128, _abi.MOE_DTYPE_INT8, OTHER, None) == _abi.MOE_OK


def test_ffn_layer_argument_errors(L):
    """moe_ffn_layer: its workspace (the block's plus the two branch inputs)
    and every error it reports before launching anything."""
    d = _real()
    T, H = 8, 2816
    wsb = L.moe_workspace_bytes(ctypes.byref(d), T)
    ws = L.moe_ffn_workspace_bytes(ctypes.byref(d), T)
    assert ws == wsb + 2 * T * H * 2
    assert L.moe_ffn_workspace_bytes(ctypes.byref(d), -1) == 0
    norms = _abi.MoeFfnNorms(FAKE, FAKE, FAKE, FAKE, FAKE, 1e-6)
    ok = dict(h=FAKE, T=T, out=FAKE + (1 << 20), ws=FAKE, ws_bytes=ws)

    def call(n=norms, w=None, dbg=None, **kw):
        a = dict(ok, **kw)
        w = w or _weights()
        return L.moe_ffn_layer(ctypes.byref(d), ctypes.byref(w), ctypes.byref(n) if n is not None else None,
                               a["h"], a["T"], a["out"], dbg, a["ws"], a["ws_bytes"], None)

    assert call(h=None) == _abi.MOE_ERR_NULL
    assert call(out=None) == _abi.MOE_ERR_NULL
    assert call(ws=None) == _abi.MOE_ERR_NULL
    assert call(out=FAKE) == _abi.MOE_ERR_SHAPE            # out aliases h
    assert call(h=FAKE + 8) == _abi.MOE_ERR_ALIGN
    assert call(ws_bytes=ws - 1) == _abi.MOE_ERR_WORKSPACE
    assert call(ws_bytes=wsb) == _abi.MOE_ERR_WORKSPACE    # the block's alone is too small
    assert call(n=_abi.MoeFfnNorms(FAKE, FAKE + 2, FAKE, FAKE, FAKE, 1e-6)) == _abi.MOE_ERR_ALIGN
    assert b"pre_moe" in L.moe_last_error()
    assert call(n=_abi.MoeFfnNorms(FAKE, FAKE, FAKE, FAKE, FAKE, -1.0)) == _abi.MOE_ERR_SHAPE
    assert call(w=_weights(layout=_abi.MOE_LAYOUT_ROWS)) == _abi.MOE_ERR_UNSUPPORTED
    # a forced path that cannot run is refused before the pre-norm launch
    dbg = _abi.MoeDebug()
    dbg.path = _abi.MOE_PATH_STREAM
    wsT = L.moe_ffn_workspace_bytes(ctypes.byref(d), 100)
    assert call(dbg=ctypes.byref(dbg), T=100, ws_bytes=wsT) == _abi.MOE_ERR_UNSUPPORTED
    # an empty batch is a valid no-op, with or without gains
    assert call(T=0, h=None, out=None, ws=None, ws_bytes=0) == _abi.MOE_OK
    assert call(n=None, T=0, h=None, out=None, ws=None, ws_bytes=0) == _abi.MOE_OK


def test_prefill_chunk_size_rule(L):
    """The chunk size of the chunked prefill ([TT] "Configurable knobs": 16384
    tokens by default, snapped to a multiple of the 1024-token sliding window,
    capped at 32768). Host arithmetic only."""
    cases = {0: 16384, -7: 16384, 1: 1024, 1023: 1024, 1024: 1024, 2047: 1024, 2048: 2048,
             5000: 4096, 16384: 16384, 16385: 16384, 32768: 32768, 40000: 32768, 2 ** 31 - 1: 32768}
    for req, want in cases.items():
        assert L.moe_prefill_chunk_tokens(req) == want, req
    d = _real()
    for req in (0, 1500, 40000):
        c = L.moe_prefill_chunk_tokens(req)
        assert L.moe_prefill_workspace_bytes(ctypes.byref(d), req) == L.moe_ffn_workspace_bytes(ctypes.byref(d), c)
    bad = _abi.MoeDims(2816, 128, 9, 704, 2112, 1e-6)
    assert L.moe_prefill_workspace_bytes(ctypes.byref(bad), 0) == 0


def test_prefill_chunked_argument_errors(L):
    """moe_prefill_chunked checks everything before it launches: the block's
    arguments, the gains (with norms), and a workspace that must hold the
    largest chunk, which is less than the whole prompt's."""
    d = _real()
    T, C = 5000, 2048
    ws_chunk = L.moe_prefill_workspace_bytes(ctypes.byref(d), C)
    ws_block = L.moe_workspace_bytes(ctypes.byref(d), C)
    assert ws_chunk < L.moe_ffn_workspace_bytes(ctypes.byref(d), T)
    norms = _abi.MoeFfnNorms(FAKE, FAKE, FAKE, FAKE, FAKE, 1e-6)
    ok = dict(h=FAKE, T=T, out=FAKE + (1 << 26), ws=FAKE, ws_bytes=ws_chunk)

    def call(n=norms, w=None, chunk=C, **kw):
        a = dict(ok, **kw)
        w = w or _weights()
        return L.moe_prefill_chunked(ctypes.byref(d), ctypes.byref(w), ctypes.byref(n) if n is not None else None,
                                     a["h"], a["T"], chunk, a["out"], a["ws"], a["ws_bytes"], None)

    assert call(h=None) == _abi.MOE_ERR_NULL
    assert call(out=None) == _abi.MOE_ERR_NULL
    assert call(ws=None) == _abi.MOE_ERR_NULL
    assert call(out=FAKE) == _abi.MOE_ERR_SHAPE              # out aliases h
    assert call(T=-1) == _abi.MOE_ERR_SHAPE
    assert call(ws=FAKE + 16) == _abi.MOE_ERR_ALIGN
    assert call(ws_bytes=ws_chunk - 1) == _abi.MOE_ERR_WORKSPACE
    assert call(ws_bytes=ws_block) == _abi.MOE_ERR_WORKSPACE  # the layer needs its branch inputs too
    assert call(chunk=4096, ws_bytes=ws_chunk) == _abi.MOE_ERR_WORKSPACE
    assert call(n=_abi.MoeFfnNorms(FAKE, FAKE, FAKE, FAKE, FAKE + 4, 1e-6)) == _abi.MOE_ERR_ALIGN
    assert b"post" in L.moe_last_error()
    assert call(w=_weights(layout=_abi.MOE_LAYOUT_ROWS)) == _abi.MOE_ERR_UNSUPPORTED
    # an empty prompt is a valid no-op
    assert call(T=0, h=None, out=None, ws=None, ws_bytes=0) == _abi.MOE_OK
    assert call(n=None, T=0, h=None, out=None, ws=None, ws_bytes=0) == _abi.MOE_OK


def test_fp8_argument_errors(L):
    """E4M3 experts: the scales are required, hidden and expert_inter are
    limited to 16384 (the per-row quantisers hold a row in registers), the
    quantiser checks its shape, and every error comes before any launch."""
    d = _real()
    T = 8
    ws = L.moe_workspace_bytes(ctypes.byref(d), T)

    def block(w, dims=d):
        return L.moe_block(ctypes.byref(dims), ctypes.byref(w), FAKE, T, FAKE + (1 << 20), None, FAKE,
                           L.moe_workspace_bytes(ctypes.byref(dims), T), None)

    fp8 = dict(expert_dtype=_abi.MOE_DTYPE_FP8)
    assert block(_weights(**fp8)) == _abi.MOE_ERR_NULL                       # scales missing
    assert b"gate_up_scale" in L.moe_last_error()
    assert block(_weights(**fp8, gate_up_scale=FAKE)) == _abi.MOE_ERR_NULL   # down_scale missing
    assert block(_weights(**fp8, gate_up_scale=FAKE + 2, down_scale=FAKE)) == _abi.MOE_ERR_ALIGN
    assert block(_weights(expert_dtype=3, gate_up_scale=FAKE, down_scale=FAKE)) == _abi.MOE_ERR_UNSUPPORTED
    wide = _abi.MoeDims(16640, 128, 8, 704, 2112, 1e-6)
    assert block(_weights(**fp8, gate_up_scale=FAKE, down_scale=FAKE), wide) == _abi.MOE_ERR_UNSUPPORTED
    assert b"16384" in L.moe_last_error()
    # the quantiser: shape and pointer checks, and an empty matrix is a no-op
    assert L.moe_quantize_fp8(FAKE, 4, 12, FAKE, FAKE, None) == _abi.MOE_ERR_SHAPE   # cols % 8
    assert L.moe_quantize_fp8(FAKE, -1, 16, FAKE, FAKE, None) == _abi.MOE_ERR_SHAPE
    assert L.moe_quantize_fp8(None, 4, 16, FAKE, FAKE, None) == _abi.MOE_ERR_NULL
    assert L.moe_quantize_fp8(FAKE, 4, 16, FAKE + 8, FAKE, None) == _abi.MOE_ERR_ALIGN
    assert L.moe_quantize_fp8(FAKE, 0, 16, FAKE, FAKE, None) == _abi.MOE_OK
    # E4M3 tiles are 1-byte tiles
    assert L.moe_tile_weights(FAKE, 16, 64, _abi.MOE_DTYPE_FP8, FAKE, None) == _abi.MOE_ERR_SHAPE  # src == dst
    assert L.moe_tile_weights(FAKE, 0, 64, _abi.MOE_DTYPE_FP8, FAKE + 64, None) == _abi.MOE_OK


def _host_layer(dims, fmt="bf16"):
    """A layer of host tensors with the shapes and dtypes dims imply."""
    import torch
    from mixture_experts_ffn_amd import LayerWeights
    H, E, I, Id = dims.hidden, dims.num_experts, dims.expert_inter, dims.dense_inter
    bf = torch.bfloat16
    ex = {"bf16": bf, "int8": torch.int8, "fp8": torch.float8_e4m3fn}[fmt]
    lw = LayerWeights(router_scale=torch.zeros(H, dtype=bf), router_w=torch.zeros((E, H), dtype=bf),
                      per_expert_scale=torch.ones(E), expert_gate_up=torch.zeros((E, 2 * I, H), dtype=ex),
                      expert_down=torch.zeros((E, H, I), dtype=ex), dense_gate_up=torch.zeros((2 * Id, H), dtype=bf),
                      dense_down=torch.zeros((H, Id), dtype=bf))
    if fmt != "bf16":
        lw.gate_up_scale, lw.down_scale = torch.ones((E, 2 * I)), torch.ones((E, H))
    return lw


def test_no_fallback_missing_library_and_host_tensors(tmp_path):
    """There is no other implementation: a missing library raises at load time,
    and host tensors are refused by the binding instead of being computed on
    the CPU."""
    import torch
    from mixture_experts_ffn_amd import BlockDims, moe_block, moe_ffn_layer, moe_prefill_chunked
    with pytest.raises(RuntimeError, match="missing"):
        _abi.load_library(str(tmp_path / "libmoe_ffn.so"))
    dims = BlockDims(512, 16, 4, 128, 384)
    lw = _host_layer(dims)
    x = torch.zeros((8, 512), dtype=torch.bfloat16)
    for call in (lambda: moe_block(dims, lw, x), lambda: moe_ffn_layer(dims, lw, None, x),
                 lambda: moe_prefill_chunked(dims, lw, None, x)):
        with pytest.raises(ValueError, match="device tensor"):
            call()


def test_binding_checks_shapes_dtypes_and_devices():
    """The C ABI receives bare pointers, so the binding checks every tensor
    against the dims before any call: a mismatch raises instead of becoming an
    out-of-bounds access on the device. Host tensors suffice: these checks come
    before the device check."""
    import dataclasses
    import torch
    from mixture_experts_ffn_amd import (BlockCall, BlockDims, FfnNorms, dense_mlp, moe_block, moe_ffn_layer,
                                         moe_quantize_int8, moe_route, moe_tile_weights)
    dims = BlockDims(256, 4, 2, 64, 64)
    bf = torch.bfloat16
    x = torch.zeros((8, 256), dtype=bf)
    good = _host_layer(dims)

    def raises(fn, match):
        with pytest.raises((ValueError, TypeError), match=match):
            fn()

    # the activations
    raises(lambda: moe_block(dims, good, torch.zeros((8, 128), dtype=bf)), r"expected \(T, 256\)")
    raises(lambda: moe_block(dims, good, torch.zeros((8, 256))), "dtype")
    raises(lambda: moe_block(dims, good, torch.zeros(256, dtype=bf)), "shape")
    raises(lambda: moe_block(dims, good, x, y=torch.zeros((8, 128), dtype=bf)), "y has shape")
    raises(lambda: moe_block(dims, good, x, y=torch.zeros((8, 256))), "y has dtype")
    # every weight against the dims
    bad = {"router_scale": torch.zeros(128, dtype=bf), "router_w": torch.zeros((4, 128), dtype=bf),
           "per_expert_scale": torch.ones(3), "logit_bias": torch.zeros(5),
           "expert_gate_up": torch.zeros((4, 64, 256), dtype=bf), "expert_down": torch.zeros((4, 256, 32), dtype=bf),
           "dense_gate_up": torch.zeros((64, 256), dtype=bf), "dense_down": torch.zeros((256, 32), dtype=bf)}
    for k, v in bad.items():
        raises(lambda: moe_block(dims, dataclasses.replace(good, **{k: v}), x), k)
    raises(lambda: moe_block(dims, dataclasses.replace(good, per_expert_scale=torch.ones(4, dtype=torch.float64)),
                             x), "per_expert_scale has dtype")
    # 1-byte experts: scales present and of the right shape; down in the same format
    q8 = _host_layer(dims, "int8")
    raises(lambda: moe_block(dims, dataclasses.replace(q8, down_scale=None), x), "down_scale")
    raises(lambda: moe_block(dims, dataclasses.replace(q8, gate_up_scale=torch.ones((4, 64))), x), "gate_up_scale")
    raises(lambda: moe_block(dims, dataclasses.replace(q8, expert_down=torch.zeros((4, 256, 64), dtype=bf)), x),
           "expert_down has dtype")
    # the router alone, the dense MLP alone, the layer
    raises(lambda: moe_route(dims, good, x, topk_idx=torch.zeros((8, 3), dtype=torch.int32)), "topk_idx")
    raises(lambda: moe_route(dims, good, x, topk_w=torch.zeros((8, 2), dtype=bf)), "topk_w")
    raises(lambda: dense_mlp(dims, good.dense_gate_up, torch.zeros((256, 128), dtype=bf), x), "dense_down")
    raises(lambda: moe_ffn_layer(dims, good, FfnNorms(post=torch.zeros(128, dtype=bf)), x), "post has shape")
    raises(lambda: moe_ffn_layer(dims, good, None, x, out=torch.zeros((4, 256), dtype=bf)), "out has shape")
    raises(lambda: BlockCall(dims, good, torch.zeros((8, 512), dtype=bf)), "shape")
    # load-time helpers
    raises(lambda: moe_quantize_int8(torch.zeros((4, 64))), "dtype")
    raises(lambda: moe_quantize_int8(torch.zeros((4, 64), dtype=bf), scale=torch.ones(3)), "scale has shape")
    raises(lambda: moe_tile_weights(torch.zeros((16, 64), dtype=bf), out=torch.zeros((16, 64), dtype=torch.int8)),
           "out has")
    # debug outputs too small for T * K
    from mixture_experts_ffn_amd.ops import _debug_outputs
    dbg = _abi.MoeDebug()
    dbg._outputs = {"topk_idx": torch.zeros(8, dtype=torch.int32)}
    raises(lambda: _debug_outputs(dbg, dims, 8), "topk_idx must hold at least 16")
    dbg._outputs = {"offsets": torch.zeros(4, dtype=torch.int32)}
    raises(lambda: _debug_outputs(dbg, dims, 8), "offsets must hold at least 5")
    dbg._outputs = {"topk_w": torch.zeros(16, dtype=torch.int32)}
    raises(lambda: _debug_outputs(dbg, dims, 8), "topk_w")
    # all tensors on one device
    if torch.cuda.is_available():
        raises(lambda: moe_block(dims, good, x.cuda()), "different devices")
