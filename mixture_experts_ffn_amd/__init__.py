"""MI355X-native hybrid MoE FFN block (Gemma-4 26B-A4B shape) on gfx950.

The compute lives in ``libmoe_ffn.so`` (hand-written HIP kernels behind the C
ABI of ``include/moe.h``); this package only marshals torch tensors to it.
"""
from ._abi import (MOE_DTYPE_BF16, MOE_DTYPE_FP8, MOE_DTYPE_INT8, MOE_LAYOUT_ROWS, MOE_LAYOUT_TILED,  # noqa: F401
                   MOE_PATH_AUTO, MOE_PATH_GROUPED, MOE_PATH_STREAM, MOE_STREAM_MAX_TOKENS,
                   load_library)
from .ops import (BlockCall, BlockDims, FfnCall, FfnNorms, LayerWeights, MoEError, dense_mlp, moe_block,  # noqa: F401
                  moe_block_noalloc,
                  moe_ffn_layer, moe_ffn_workspace_bytes, moe_prefill_chunk_tokens, moe_prefill_chunked,
                  moe_prefill_workspace_bytes, moe_quantize_fp8, moe_quantize_int8, moe_route, moe_tile_weights,
                  moe_workspace_bytes, new_debug, tile_layer)
