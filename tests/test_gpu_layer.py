"""GPU MoE layer parity (route -> gate/up -> SiLU*up -> down -> combine) against
the fp64 oracle, in all three formats, at small shapes and at the full layer
shape (256 experts, d_model 4096, d_ff 2048, top-6) for B = 1 and B = 8.

Invariants: run-to-run bitwise determinism, identical tokens give identical
rows (and 6 unique experts), and a token's result does not depend on the
batch width (B=8 row t == B=1 run of token t, bitwise)."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import Layer, assert_parity

pytestmark = pytest.mark.gpu

_LAYERS = {}


def layer(fmt, E, D, F, k=6, seed=0x5EED, lid=0):
    key = (fmt, E, D, F, k, seed, lid)
    if key not in _LAYERS:
        if len(_LAYERS) > 3:  # keep device memory bounded across the module
            _LAYERS.clear()
            torch.cuda.empty_cache()
        _LAYERS[key] = Layer(fmt, seed, lid, E, D, F, k)
    return _LAYERS[key]


def _parity(L, xb, what):
    y, idx, gw = L.run(xb)
    yo, io, go = L.oracle(xb)
    assert np.array_equal(idx, io), f"{what}: routing differs"
    assert np.max(np.abs(gw - go)) <= 1e-6
    return assert_parity(y, yo, what=what), y


@pytest.mark.parametrize("fmt", ["mxfp4", "q2k", "int4g32"])
@pytest.mark.parametrize("B", [1, 3, 8])
def test_layer_small(fmt, B):
    L = layer(fmt, 32, 512, 256, 6, seed=11)
    xb = synth.token_bf16(500 + B, B, 512)
    _parity(L, xb, f"{fmt} small B={B}")


def test_layer_multi_launch_fallback_shape():
    # d_model 8192 has more MXFP4 blocks per row than the single-launch
    # kernel keeps per lane, so the layer runs as separate launches.
    L = layer("mxfp4", 16, 8192, 256, 6, seed=13)
    for B in (1, 8):
        _parity(L, synth.token_bf16(700 + B, B, 8192), f"fallback B={B}")


def test_layer_small_ragged_topk_and_experts():
    L = layer("mxfp4", 10, 96, 64, 3, seed=12)
    for B in (1, 4, 8):
        _parity(L, synth.token_bf16(600 + B, B, 96), f"ragged B={B}")


@pytest.mark.parametrize("B", [1, 8])
def test_layer_full_mxfp4(B):
    L = layer("mxfp4", 256, 4096, 2048)
    err, y = _parity(L, synth.token_bf16(1000 + B, B, 4096), f"mxfp4 full B={B}")
    print(f"mxfp4 layer B={B}: max rel-inf err {err:.3e}")


@pytest.mark.parametrize("fmt", ["q2k", "int4g32"])
@pytest.mark.parametrize("B", [1, 8])
def test_layer_full_other_formats(fmt, B):
    L = layer(fmt, 256, 4096, 2048)
    err, y = _parity(L, synth.token_bf16(2000 + B, B, 4096), f"{fmt} full B={B}")
    print(f"{fmt} layer B={B}: max rel-inf err {err:.3e}")


def _single_launch(L, B):
    import quantized_moe_decode_route_amd as moe
    x = torch.zeros((B, L.D), dtype=torch.int16, device="cuda")
    y = torch.empty((B, L.D), dtype=torch.float32, device="cuda")
    return moe.moe_layer_decode_traced(L.desc, x, y, L.workspace(B)) is not None


def test_layer_invariants_full_shape():
    L = layer("mxfp4", 256, 4096, 2048)
    assert _single_launch(L, 1) and _single_launch(L, 8), "full layer shape should run as one launch"
    x8 = synth.token_bf16(3000, 8, 4096)
    ws = L.workspace(8)
    y8a, i8a, _ = L.run(x8, ws)
    y8b, i8b, _ = L.run(x8, ws)
    assert np.array_equal(y8a, y8b) and np.array_equal(i8a, i8b)          # determinism
    for t in range(8):                                                       # width invariance
        y1, i1, _ = L.run(x8[t:t + 1])
        assert np.array_equal(i1[0], i8a[t])
        assert np.array_equal(y1[0], y8a[t]), f"token {t}: B=8 row differs from B=1"
    xs = np.repeat(x8[:1], 8, axis=0)                                        # identical tokens
    ys, is_, _ = L.run(xs)
    assert all(np.array_equal(ys[0], ys[t]) for t in range(8))
    assert len(np.unique(is_)) == 6
    assert np.array_equal(ys[0], y8a[0])
