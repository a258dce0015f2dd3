"""The no-allocation layer entry point (moe_layer_decode_noalloc), whose
workspace is the library's static per-device scratch, against
moe_layer_decode with a caller workspace: the same kernels on the same
inputs, so the outputs, expert indices and gate weights must agree bit for
bit.  Two calls in a row, the second with fewer tokens (the scratch keeps
the first call's contents), at the full layer shape (256 experts, 4096 x
2048, MXFP4, matrix-core down layout).  It must pass alone in a fresh
process (the first call sets the scratch up) and after other tests."""
import numpy as np
import pytest
import torch

import quantized_moe_decode_route_amd as moe
import synth
from gpu_helpers import Layer, dev, host

pytestmark = pytest.mark.gpu


def _with_workspace(L, xb):
    return L.run(xb)


def _noalloc(L, xb):
    B = xb.shape[0]
    y = torch.full((B, L.D), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((B, L.k), -1, dtype=torch.int32, device="cuda")
    gw = torch.full((B, L.k), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_layer_decode_noalloc(L.desc, dev(xb), y, idx, gw)
    torch.cuda.synchronize()
    return host(y), host(idx), host(gw)


def test_noalloc_matches_workspace_entry_two_calls():
    L = Layer("mxfp4", 0x5EED + 80, 0, 256, 4096, 2048, 6, down_layout="mfma16")
    x8 = synth.token_bf16(8800, 8, 4096)
    x3 = synth.token_bf16(8900, 3, 4096)
    for xb in (x8, x3):   # second call smaller
        y_ref, i_ref, g_ref = _with_workspace(L, xb)
        y, idx, gw = _noalloc(L, xb)
        assert np.array_equal(idx, i_ref)
        assert np.array_equal(gw.view(np.uint32), g_ref.view(np.uint32))
        assert np.array_equal(y.view(np.uint32), y_ref.view(np.uint32)), f"B={xb.shape[0]}"
    # once more at B = 1 after the smaller call, on another layer format
    Q = Layer("q2k", 0x5EED + 81, 0, 32, 512, 256, 6, down_layout="tile256")
    x1 = synth.token_bf16(8950, 1, 512)
    y_ref, i_ref, _ = _with_workspace(Q, x1)
    y, idx, _ = _noalloc(Q, x1)
    assert np.array_equal(idx, i_ref) and np.array_equal(y.view(np.uint32), y_ref.view(np.uint32))


def test_noalloc_rejects_a_call_beyond_the_scratch():
    L = Layer("mxfp4", 0x5EED + 82, 0, 16, 8192, 512, 6)
    x = torch.zeros((8, 8192), dtype=torch.int16, device="cuda")
    y = torch.empty((8, 8192), dtype=torch.float32, device="cuda")
    with pytest.raises(moe.MoeError) as err:
        moe.moe_layer_decode_noalloc(L.desc, x, y)
    assert err.value.status == moe.MOE_ERR_SCRATCH
