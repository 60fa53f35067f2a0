"""ctypes view of include/moe.h and loading of libmoe_ffn.so.

The structures mirror the C declarations field for field. Loading fails loudly
when the library has not been built: there is no other implementation.
"""
from __future__ import annotations

import ctypes
import os

LIB_NAME = "libmoe_ffn.so"
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)
HEADER_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe.h")

MOE_OK = 0
MOE_ERR_NULL = -1
MOE_ERR_SHAPE = -2
MOE_ERR_UNSUPPORTED = -3
MOE_ERR_WORKSPACE = -4
MOE_ERR_HIP = -5
MOE_ERR_ALIGN = -6
STATUS_NAMES = {
    MOE_OK: "MOE_OK", MOE_ERR_NULL: "MOE_ERR_NULL", MOE_ERR_SHAPE: "MOE_ERR_SHAPE",
    MOE_ERR_UNSUPPORTED: "MOE_ERR_UNSUPPORTED", MOE_ERR_WORKSPACE: "MOE_ERR_WORKSPACE",
    MOE_ERR_HIP: "MOE_ERR_HIP", MOE_ERR_ALIGN: "MOE_ERR_ALIGN",
}

MOE_MAX_TOKENS = 1 << 22
MOE_MAX_EXPERTS = 256
MOE_MAX_TOPK = 8
MOE_DTYPE_BF16 = 0
MOE_DTYPE_INT8 = 1
MOE_DTYPE_FP8 = 2
MOE_PATH_AUTO = 0
MOE_PATH_STREAM = 1
MOE_PATH_GROUPED = 2
MOE_STREAM_MAX_TOKENS = 64
MOE_MAX_STAGES = 8
MOE_LAYOUT_ROWS = 0
MOE_LAYOUT_TILED = 1


class MoeDims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("expert_inter", ctypes.c_int32),
                ("dense_inter", ctypes.c_int32), ("rms_eps", ctypes.c_float)]


class MoeWeights(ctypes.Structure):
    _fields_ = [("router_scale", ctypes.c_void_p), ("router_w", ctypes.c_void_p),
                ("per_expert_scale", ctypes.c_void_p), ("logit_bias", ctypes.c_void_p),
                ("expert_gate_up", ctypes.c_void_p), ("expert_down", ctypes.c_void_p),
                ("expert_dtype", ctypes.c_int32), ("gate_up_scale", ctypes.c_void_p),
                ("down_scale", ctypes.c_void_p), ("dense_gate_up", ctypes.c_void_p),
                ("dense_down", ctypes.c_void_p), ("layout", ctypes.c_int32)]


class MoeDebug(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("topk_idx", ctypes.c_void_p),
                ("topk_w", ctypes.c_void_p), ("counts", ctypes.c_void_p),
                ("offsets", ctypes.c_void_p), ("perm_token", ctypes.c_void_p),
                ("inv_row", ctypes.c_void_p),
                ("stage_event", ctypes.c_void_p * (MOE_MAX_STAGES + 1)),
                ("path_taken", ctypes.c_int32), ("n_stages", ctypes.c_int32),
                ("stage_name", ctypes.c_char_p * MOE_MAX_STAGES)]


class MoeFfnNorms(ctypes.Structure):
    _fields_ = [("pre_dense", ctypes.c_void_p), ("pre_moe", ctypes.c_void_p),
                ("post_dense", ctypes.c_void_p), ("post_moe", ctypes.c_void_p),
                ("post", ctypes.c_void_p), ("eps", ctypes.c_float)]


MOE_NOALLOC_SCRATCH_BYTES = 32 << 20

EXPORTS = ("moe_workspace_bytes", "moe_route", "moe_block", "moe_block_noalloc", "dense_mlp",
           "moe_ffn_workspace_bytes", "moe_ffn_layer",
           "moe_prefill_chunk_tokens", "moe_prefill_workspace_bytes", "moe_prefill_chunked",
           "moe_quantize_int8", "moe_quantize_fp8", "moe_tile_weights", "moe_last_error")

_lib = None


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libmoe_ffn.so and declare the signatures of include/moe.h."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(
            f"{p} is missing: build the HIP library first (python -m mixture_experts_ffn_amd.build)")
    lib = ctypes.CDLL(p)
    P = ctypes.POINTER
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.moe_workspace_bytes.argtypes = [P(MoeDims), i32]
    lib.moe_workspace_bytes.restype = sz
    lib.moe_route.argtypes = [P(MoeDims), P(MoeWeights), vp, i32, vp, vp, vp, sz, vp]
    lib.moe_route.restype = ctypes.c_int
    lib.moe_block.argtypes = [P(MoeDims), P(MoeWeights), vp, i32, vp, P(MoeDebug), vp, sz, vp]
    lib.moe_block.restype = ctypes.c_int
    lib.moe_block_noalloc.argtypes = [P(MoeDims), P(MoeWeights), vp, i32, vp, P(MoeDebug), vp]
    lib.moe_block_noalloc.restype = ctypes.c_int
    lib.dense_mlp.argtypes = [P(MoeDims), vp, vp, vp, i32, vp, vp, sz, vp]
    lib.dense_mlp.restype = ctypes.c_int
    lib.moe_ffn_workspace_bytes.argtypes = [P(MoeDims), i32]
    lib.moe_ffn_workspace_bytes.restype = sz
    lib.moe_ffn_layer.argtypes = [P(MoeDims), P(MoeWeights), P(MoeFfnNorms), vp, i32, vp, P(MoeDebug), vp, sz,
                                  vp]
    lib.moe_ffn_layer.restype = ctypes.c_int
    lib.moe_prefill_chunk_tokens.argtypes = [i32]
    lib.moe_prefill_chunk_tokens.restype = i32
    lib.moe_prefill_workspace_bytes.argtypes = [P(MoeDims), i32]
    lib.moe_prefill_workspace_bytes.restype = sz
    lib.moe_prefill_chunked.argtypes = [P(MoeDims), P(MoeWeights), P(MoeFfnNorms), vp, i32, i32, vp, vp, sz, vp]
    lib.moe_prefill_chunked.restype = ctypes.c_int
    lib.moe_quantize_int8.argtypes = [vp, i64, i32, vp, vp, vp]
    lib.moe_quantize_int8.restype = ctypes.c_int
    lib.moe_quantize_fp8.argtypes = [vp, i64, i32, vp, vp, vp]
    lib.moe_quantize_fp8.restype = ctypes.c_int
    lib.moe_tile_weights.argtypes = [vp, i64, i32, i32, vp, vp]
    lib.moe_tile_weights.restype = ctypes.c_int
    lib.moe_last_error.argtypes = []
    lib.moe_last_error.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib
