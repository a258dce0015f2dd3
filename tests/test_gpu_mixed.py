"""Per-family precision on the GPU: gate and up in one format, the down
projection in Q2_K, as in the pages' recipe ("Mixed-precision compression of
DeepSeek-V4-Flash", "The recipe": routed gate/up at 2 bits, down at Q2_K;
IQ2_XXS's codebook is not on the pages, so MXFP4 or INT4 group-32 stand in
for the gate/up format).  Parity against the fp64 oracle composed with the
same per-projection formats, on both launch paths, at every batch width, and
a Q2_K layer stack."""
import numpy as np
import pytest
import torch

import oracle
import quantized_moe_decode_route_amd as moe
import synth
from gpu_helpers import Layer, assert_parity, dev, host

pytestmark = pytest.mark.gpu

PAIRS = [("mxfp4", "q2k"), ("int4g32", "q2k")]


def _single_launch(L, B):
    x = torch.zeros((B, L.D), dtype=torch.int16, device="cuda")
    y = torch.empty((B, L.D), dtype=torch.float32, device="cuda")
    return moe.moe_layer_decode_traced(L.desc, x, y, L.workspace(B)) is not None


def _parity(L, xb, what):
    y, idx, gw = L.run(xb)
    yo, io, go = L.oracle(xb)
    assert np.array_equal(idx, io), f"{what}: routing differs"
    assert np.max(np.abs(gw - go)) <= 1e-6
    return assert_parity(y, yo, what=what)


@pytest.mark.parametrize("layout", ["rows", "tile256"])
@pytest.mark.parametrize("fmt,dfmt", PAIRS)
def test_mixed_small(fmt, dfmt, layout):
    # d_ff 512: each of 8 XCD slices holds one whole 64-column Q2_K unit
    L = Layer(fmt, 0x91, 0, 32, 512, 512, 6, down_layout=layout, down_fmt=dfmt)
    assert _single_launch(L, 1) and _single_launch(L, 8)
    for B in (1, 3, 8):
        _parity(L, synth.token_bf16(9100 + B, B, 512), f"{fmt}+{dfmt} B={B} {layout}")


@pytest.mark.parametrize("fmt,dfmt", PAIRS)
def test_mixed_every_width(fmt, dfmt):
    L = Layer(fmt, 0x92, 0, 32, 512, 512, 6, down_layout="tile256", down_fmt=dfmt)
    x8 = synth.token_bf16(9200, 8, 512)
    ws = L.workspace(8)
    ones = [L.run(x8[t:t + 1], ws) for t in range(8)]
    for B in range(2, 9):
        y, idx, _ = L.run(x8[:B], ws)
        for t in range(B):
            assert np.array_equal(idx[t], ones[t][1][0])
            assert np.array_equal(y[t].view(np.uint32), ones[t][0][0].view(np.uint32)), f"B={B} token {t}"


def test_mixed_multi_launch_fallback():
    # d_model 8192 exceeds what the single-launch kernel keeps per lane
    L = Layer("mxfp4", 0x93, 0, 16, 8192, 512, 6, down_fmt="q2k")
    assert not _single_launch(L, 1)
    for B in (1, 8):
        _parity(L, synth.token_bf16(9300 + B, B, 8192), f"fallback mxfp4+q2k B={B}")


@pytest.mark.parametrize("fmt,dfmt", PAIRS)
@pytest.mark.parametrize("B", [1, 8])
def test_mixed_full_shape(fmt, dfmt, B):
    L = Layer(fmt, 0x94, 0, 256, 4096, 2048, 6, down_layout="tile256", down_fmt=dfmt)
    assert _single_launch(L, B)
    err = _parity(L, synth.token_bf16(9400 + B, B, 4096), f"{fmt}+{dfmt} full B={B}")
    print(f"{fmt}+{dfmt} layer B={B}: max rel-inf err {err:.3e}")
    del L
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt,dfmt", [("q2k", "q2k"), ("mxfp4", "q2k")])
@pytest.mark.parametrize("B", [1, 8])
def test_stack_q2k_teacher_forced(fmt, dfmt, B):
    """A Q2_K (and a mixed) layer stack, checked layer by layer against the
    oracle fed the GPU's own residual state; the whole stack in one call
    gives the same bits as layer-by-layer calls."""
    E, D, F, n_layers = 32, 512, 512, 3
    layers = [Layer(fmt, 0x95, l, E, D, F, 6, down_layout="tile256", down_fmt=dfmt) for l in range(n_layers)]
    h0 = synth.f32_from_bf16_bits(synth.token_bf16(9500 + B, B, D))
    ws = torch.empty(moe.moe_stack_workspace_bytes(B, D, F, E, 6), dtype=torch.uint8, device="cuda")
    moe.moe_workspace_init(ws)
    hs = [h0]
    for l in range(n_layers):
        hin = dev(hs[-1])
        hout = torch.empty_like(hin)
        moe.moe_stack_decode([layers[l].desc], hin, hout, ws)
        torch.cuda.synchronize()
        hs.append(host(hout))
    for l in range(n_layers):
        xl = oracle.rmsnorm_bf16(hs[l].astype(np.float64))
        y, _, _ = layers[l].oracle(xl)
        assert_parity(hs[l + 1].astype(np.float64) - hs[l].astype(np.float64), y, what=f"layer {l}")
    hin = dev(h0)
    hout = torch.empty_like(hin)
    moe.moe_stack_decode([L.desc for L in layers], hin, hout, ws)
    torch.cuda.synchronize()
    assert np.array_equal(host(hout), hs[-1])
