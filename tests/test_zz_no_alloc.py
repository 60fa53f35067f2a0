"""moe_block_noalloc, the entry point that allocates nothing, through the C
ABI: its output and routing equal moe_block's (with a workspace of its own)
bit for bit, on two calls in a row, the second with a smaller batch, so that
the second call runs on the scratch array the first one left behind; and a
batch larger than the array is refused before anything is launched."""
import numpy as np
import pytest
import torch

import moe_synth
from mixture_experts_ffn_amd import (MOE_PATH_AUTO, MOE_PATH_GROUPED, MOE_PATH_STREAM, MoEError, moe_block,
                                     moe_block_noalloc, moe_workspace_bytes, new_debug)
from mixture_experts_ffn_amd._abi import MOE_NOALLOC_SCRATCH_BYTES
from gpu_util import bf16_dev, dims_of, upload

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda:0")


def _both(dims, lw, xd, path, K):
    """(y, topk_idx) of moe_block and of moe_block_noalloc on the same batch."""
    T = xd.shape[0]
    out = []
    for noalloc in (False, True):
        idx = torch.full((T, K), -1, dtype=torch.int32, device=xd.device)
        dbg = new_debug(path, topk_idx=idx)
        y = torch.full((T, dims.hidden), 7.0, dtype=torch.bfloat16, device=xd.device)
        if noalloc:
            moe_block_noalloc(dims, lw, xd, y, debug=dbg)
        else:
            moe_block(dims, lw, xd, y=y, debug=dbg)
        torch.cuda.synchronize()
        out.append((y, idx, dbg.path_taken))
    return out


@pytest.mark.parametrize("name,T1,T2,path", [
    ("tiny", 64, 5, MOE_PATH_AUTO),          # streaming path, then a smaller streaming batch
    ("tiny", 300, 100, MOE_PATH_GROUPED),    # grouped path twice
    ("decode", 40, 8, MOE_PATH_STREAM),      # the real shape, multi-token then plain decode
    ("decode", 300, 65, MOE_PATH_GROUPED),   # the real shape, grouped
])
def test_noalloc_matches_moe_block(dev, name, T1, T2, path):
    wl = moe_synth.WORKLOADS[name]
    s = wl.shape
    dims = dims_of(s)
    say(f"case: moe_block_noalloc {name} T={T1} then T={T2} path={path}")
    assert moe_workspace_bytes(dims, T1) <= MOE_NOALLOC_SCRATCH_BYTES
    w = moe_synth.make_weights(s, wl.seed, wl.skew)
    lw = upload(w, dev)
    x = moe_synth.make_tokens(s, wl.seed, T1)
    xd1 = bf16_dev(x, dev)
    xd2 = bf16_dev(x[::-1][:T2].copy(), dev)  # other tokens, fewer of them
    for xd in (xd1, xd2):
        (ya, ia, pa), (yb, ib, pb) = _both(dims, lw, xd, path, s.top_k)
        assert pa == pb
        assert torch.equal(ia, ib), "routing differs"
        assert torch.equal(ya.view(torch.int16), yb.view(torch.int16)), "output differs"
        say(f"  T={xd.shape[0]} path {pb}: identical")


def test_noalloc_refuses_batches_beyond_its_scratch(dev):
    wl = moe_synth.WORKLOADS["decode"]
    s = wl.shape
    dims = dims_of(s)
    T = 2048
    assert moe_workspace_bytes(dims, T) > MOE_NOALLOC_SCRATCH_BYTES
    say(f"case: moe_block_noalloc refuses T={T}")
    lw = upload(moe_synth.make_weights(s, wl.seed, wl.skew), dev)
    x = torch.zeros((T, s.hidden), dtype=torch.bfloat16, device=dev)
    y = torch.full_like(x, 3.0)
    with pytest.raises(MoEError, match="WORKSPACE"):
        moe_block_noalloc(dims, lw, x, y)
    torch.cuda.synchronize()
    assert bool((y == 3.0).all()), "nothing may be written when the call is refused"
    # an empty batch is a no-op
    moe_block_noalloc(dims, lw, x[:0], y[:0])
