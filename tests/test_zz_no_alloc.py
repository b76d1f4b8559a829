"""moe_layer_decode_noalloc (static scratch, allocates nothing) against
moe_layer_decode (caller workspace): the same kernels, so the same bits, on
consecutive calls of different sizes that share the static array."""

import numpy as np
import pytest
import torch

import synth
import bit_weight_only_moe_amd as moe

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def with_workspace(L, x, res, T, k):
    nws = moe.moe_layer_decode_workspace_size(L, T)
    ws = torch.zeros(nws, dtype=torch.uint8, device=DEV)
    y = torch.empty_like(x)
    ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    moe.moe_layer_decode(L, x, res, T, y, ids, w, ws, nws)
    return y, ids, w


def without_workspace(L, x, res, T, k):
    y = torch.empty_like(x)
    ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    moe.moe_layer_decode_noalloc(L, x, res, T, y, ids, w)
    return y, ids, w


# bf16 weights: several tokens take the composed kernels, one token the fused ones, both on
# the same static array
@pytest.mark.parametrize("fmt,sizes", [(1, (16, 4)), (2, (8, 1)), (1, (64, 1, 5)), (4, (16, 1))])
def test_noalloc_matches_workspace_path(fmt, sizes):
    """Consecutive calls on the shared static array, each smaller than the one
    before and differently routed, equal moe_layer_decode on a fresh workspace
    bit for bit (ids, weights, outputs)."""
    print("noalloc", fmt, sizes, flush=True)
    H, I, E, k = 2048, 768, 256, 6
    layer = synth.make_layer(fmt, H, I, E, k, 300 + fmt, DEV)
    L = moe.Layer(layer)
    assert moe.moe_layer_decode_noalloc_max_bytes() >= moe.moe_layer_decode_workspace_size(L, 64)
    for n, T in enumerate(sizes):
        x = synth.make_tokens(T, H, 310 + 7 * n + T, DEV)
        res = synth.make_tokens(T, H, 320 + 7 * n + T, DEV)
        got = without_workspace(L, x, res, T, k)
        torch.cuda.synchronize()
        ref = with_workspace(L, x, res, T, k)
        torch.cuda.synchronize()
        assert torch.equal(got[1], ref[1]), (T, "ids")
        assert torch.equal(got[2], ref[2]), (T, "weights")
        assert torch.equal(got[0].view(torch.int16), ref[0].view(torch.int16)), (T, "y")
        assert torch.isfinite(got[0].float()).all()


def test_noalloc_without_shared_expert_or_outputs():
    """No shared expert, no ids/weights outputs, no residual."""
    print("noalloc variants", flush=True)
    H, I, E, k, T = 256, 128, 32, 6, 3
    layer = synth.make_layer(2, H, I, E, k, 330, DEV, shared=False)
    L = moe.Layer(layer)
    x = synth.make_tokens(T, H, 331, DEV)
    y = torch.empty_like(x)
    moe.moe_layer_decode_noalloc(L, x, None, T, y)
    torch.cuda.synchronize()
    ref = with_workspace(L, x, None, T, k)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), ref[0].view(torch.int16))
