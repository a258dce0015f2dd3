"""GPU stacked decode: the inter-layer RMSNorm (bit-exact bfloat16 with the
oracle) and the residual stream through several layers, checked layer by
layer with teacher forcing (each layer's norm output is re-derived by the
oracle from the GPU's residual, then that layer's update is compared)."""
import numpy as np
import pytest
import torch

import oracle
import quantized_moe_decode_route_amd as moe
import synth
from gpu_helpers import Layer, assert_parity, dev, host

pytestmark = pytest.mark.gpu


def test_rmsnorm_bit_exact():
    rng = np.random.default_rng(1)
    for D, scale in ((4096, 1e11), (256, 1.0), (96, 3e-5)):
        h = (rng.standard_normal((8, D)) * scale).astype(np.float32)
        x = torch.empty((8, D), dtype=torch.int16, device="cuda")
        moe.moe_rmsnorm_bf16(dev(h), x, 1e-6)
        torch.cuda.synchronize()
        assert np.array_equal(host(x, np.uint16), oracle.rmsnorm_bf16(h.astype(np.float64), 1e-6))


@pytest.mark.parametrize("B", [1, 8])
def test_stack_teacher_forced(B):
    E, D, F, n_layers = 32, 512, 256, 4
    layers = [Layer("mxfp4", 21, l, E, D, F, 6) for l in range(n_layers)]
    x0 = synth.token_bf16(77 + B, B, D)
    h0 = synth.f32_from_bf16_bits(x0)
    ws = torch.empty(moe.moe_stack_workspace_bytes(B, D, F, E, 6), dtype=torch.uint8, device="cuda")
    moe.moe_workspace_init(ws)
    hs = [h0]
    # run the stack one layer at a time to observe every residual state
    for l in range(n_layers):
        hin = dev(hs[-1])
        hout = torch.empty_like(hin)
        moe.moe_stack_decode([layers[l].desc], hin, hout, ws)
        torch.cuda.synchronize()
        hs.append(host(hout))
    for l in range(n_layers):
        xl = oracle.rmsnorm_bf16(hs[l].astype(np.float64))
        y, _, _ = layers[l].oracle(xl)
        upd = hs[l + 1].astype(np.float64) - hs[l].astype(np.float64)
        assert_parity(upd, y, tol=1e-4, what=f"layer {l}")
    # the whole stack in one call gives the same bits as layer-by-layer calls
    hin = dev(h0)
    hout = torch.empty_like(hin)
    moe.moe_stack_decode([L.desc for L in layers], hin, hout, ws)
    torch.cuda.synchronize()
    assert np.array_equal(host(hout), hs[-1])


def test_stack_full_shape_three_layers():
    D, F, E = 4096, 2048, 256
    layers = [Layer("mxfp4", 0x5EED + 4, l, E, D, F, 6) for l in range(3)]
    x0 = synth.token_bf16(4000, 1, D)
    h0 = synth.f32_from_bf16_bits(x0)
    ws = torch.empty(moe.moe_stack_workspace_bytes(1, D, F, E, 6), dtype=torch.uint8, device="cuda")
    moe.moe_workspace_init(ws)
    hs = [h0]
    for l in range(3):
        hin = dev(hs[-1])
        hout = torch.empty_like(hin)
        moe.moe_stack_decode([layers[l].desc], hin, hout, ws)
        torch.cuda.synchronize()
        hs.append(host(hout))
    for l in range(3):
        xl = oracle.rmsnorm_bf16(hs[l].astype(np.float64))
        y, _, _ = layers[l].oracle(xl)
        assert_parity(hs[l + 1].astype(np.float64) - hs[l].astype(np.float64), y, what=f"full layer {l}")
    del layers
    torch.cuda.empty_cache()
