"""GPU MoE layer parity (route -> gate/up -> SiLU*up -> down -> combine) against
the fp64 oracle, in all three formats, at small shapes and at the full layer
shape (256 experts, d_model 4096, d_ff 2048, top-6) for B = 1 and B = 8.

The down-projection layouts (row-major as published, 256-column tiles, and
for MXFP4 the tiles ordered for the matrix cores) are covered; the
full-shape Q2_K and INT4 runs use the tiled layout.

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


def layer(fmt, E, D, F, k=6, seed=0x5EED, lid=0, down_layout="rows"):
    key = (fmt, E, D, F, k, seed, lid, down_layout)
    if key not in _LAYERS:
        if len(_LAYERS) > 2:  # keep device memory bounded across the module
            _LAYERS.clear()
            torch.cuda.empty_cache()
        _LAYERS[key] = Layer(fmt, seed, lid, E, D, F, k, down_layout=down_layout)
    return _LAYERS[key]


def _parity(L, xb, what):
    y, idx, gw = L.run(xb)
    yo, io, go = L.oracle(xb)
    assert np.array_equal(idx, io), f"{what}: routing differs"
    assert np.max(np.abs(gw - go)) <= 1e-6
    return assert_parity(y, yo, what=what), y


FMT_LAYOUTS = [(f, l) for f in ("mxfp4", "q2k", "int4g32") for l in ("rows", "tile256")] + [("mxfp4", "mfma16")]
MX_LAYOUTS = ["rows", "tile256", "mfma16"]


@pytest.mark.parametrize("fmt,layout", FMT_LAYOUTS)
@pytest.mark.parametrize("B", [1, 3, 8])
def test_layer_small(fmt, B, layout):
    L = layer(fmt, 32, 512, 256, 6, seed=11, down_layout=layout)
    xb = synth.token_bf16(500 + B, B, 512)
    _parity(L, xb, f"{fmt} small B={B} {layout}")


@pytest.mark.parametrize("layout", MX_LAYOUTS)
def test_layer_small_several_tiles(layout):
    # d_ff 1024: four 256-column tiles per down row (two per XCD slice on an
    # 8-XCD chip would need d_ff 4096; here slices are smaller than a tile)
    L = layer("mxfp4", 24, 256, 1024, 4, seed=21, down_layout=layout)
    for B in (1, 5):
        _parity(L, synth.token_bf16(550 + B, B, 256), f"d_ff 1024 B={B} {layout}")


@pytest.mark.parametrize("layout", MX_LAYOUTS)
def test_layer_multi_launch_fallback_shape(layout):
    # d_model 8192 has more MXFP4 blocks per row than the single-launch
    # kernel keeps per lane, so the layer runs as separate launches.
    L = layer("mxfp4", 16, 8192, 512, 6, seed=13, down_layout=layout)
    assert not _single_launch(L, 1)
    for B in (1, 8):
        _parity(L, synth.token_bf16(700 + B, B, 8192), f"fallback B={B} {layout}")


def test_layer_small_ragged_topk_and_experts():
    L = layer("mxfp4", 10, 96, 64, 3, seed=12)
    for B in (1, 4, 8):
        _parity(L, synth.token_bf16(600 + B, B, 96), f"ragged B={B}")


@pytest.mark.parametrize("layout", MX_LAYOUTS)
@pytest.mark.parametrize("B", [1, 8])
def test_layer_full_mxfp4(B, layout):
    L = layer("mxfp4", 256, 4096, 2048, down_layout=layout)
    err, y = _parity(L, synth.token_bf16(1000 + B, B, 4096), f"mxfp4 full B={B} {layout}")
    print(f"mxfp4 layer B={B} {layout}: max rel-inf err {err:.3e}")


@pytest.mark.parametrize("fmt", ["q2k", "int4g32"])
@pytest.mark.parametrize("B", [1, 8])
def test_layer_full_other_formats(fmt, B):
    L = layer(fmt, 256, 4096, 2048, down_layout="tile256")
    err, y = _parity(L, synth.token_bf16(2000 + B, B, 4096), f"{fmt} full B={B} tile256")
    print(f"{fmt} layer B={B} tile256: max rel-inf err {err:.3e}")


def _single_launch(L, B):
    import quantized_moe_decode_route_amd as moe
    x = torch.zeros((B, L.D), dtype=torch.int16, device="cuda")
    y = torch.empty((B, L.D), dtype=torch.float32, device="cuda")
    return moe.moe_layer_decode_traced(L.desc, x, y, L.workspace(B)) is not None


@pytest.mark.parametrize("layout", MX_LAYOUTS)
def test_layer_invariants_full_shape(layout):
    L = layer("mxfp4", 256, 4096, 2048, down_layout=layout)
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


def test_traced_records_stay_in_bounds():
    """The traced entry point writes exactly MOE_TRACE_FIELDS words per
    workgroup: rows past the last workgroup keep their sentinel, time stamps
    of a workgroup do not decrease, and the XCD field is a small index."""
    import ctypes

    import quantized_moe_decode_route_amd as moe
    L = layer("mxfp4", 32, 512, 256, 6, seed=11)
    x = torch.from_numpy(synth.token_bf16(77, 2, 512).view(np.int16)).to("cuda")
    y = torch.empty((2, 512), dtype=torch.float32, device="cuda")
    ws = L.workspace(2)
    nb = ctypes.c_int(0)
    lib = moe.lib()
    args = (ctypes.byref(L.desc), x.data_ptr(), 2, y.data_ptr(), ws.data_ptr(), ws.numel())
    assert lib.moe_layer_decode_traced(*args, None, ctypes.byref(nb), None) == 0
    assert nb.value > 0
    guard = 4
    tr = torch.full((nb.value + guard, moe.TRACE_FIELDS), -1, dtype=torch.int64, device="cuda")
    tr[:nb.value].zero_()
    stream = torch.cuda.current_stream().cuda_stream
    assert lib.moe_layer_decode_traced(*args, tr.data_ptr(), ctypes.byref(nb), stream) == 0
    torch.cuda.synchronize()
    t = tr.cpu().numpy()
    assert (t[nb.value:] == -1).all(), "trace writes past the last workgroup's record"
    stamps = t[:nb.value, :11]
    assert (stamps > 0).all() and (np.diff(stamps, axis=1) >= 0).all()
    assert ((t[:nb.value, 6] <= t[:nb.value, 11]) & (t[:nb.value, 11] <= t[:nb.value, 12])
            & (t[:nb.value, 12] <= t[:nb.value, 7])).all()
    assert (t[:nb.value, 14] < 16).all()


def _extreme_exponents(proj, e, b):
    """A quarter of the blocks of every MXFP4 projection get scale bytes 0, 1
    or 2 (2^-127 .. 2^-125); for the down projection another eighth get
    160..170, large but with every result finite in fp32."""
    blk = b.reshape(-1, 17)
    rng = np.random.default_rng(1000 * proj + e)
    pick = rng.random(blk.shape[0])
    blk[pick < 0.25, 0] = rng.integers(0, 3, size=int((pick < 0.25).sum()))
    if proj == synth.PROJ_DOWN:
        big = (pick >= 0.25) & (pick < 0.375)
        blk[big, 0] = rng.integers(160, 171, size=int(big.sum()))
    return blk.reshape(-1)


@pytest.mark.parametrize("layout", MX_LAYOUTS)
@pytest.mark.parametrize("B", [1, 8])
def test_layer_e8m0_extremes(layout, B):
    """Tiny and large E8M0 scale bytes through the single-launch layer (the
    gate/up conversion multiplies by the subnormal 2^-127 for byte 0, the
    matrix-core down path passes the byte as the MFMA A scale)."""
    L = Layer("mxfp4", 0x5EED + 70, 0, 16, 512, 256, 6, down_layout=layout, mutate=_extreme_exponents)
    assert _single_launch(L, B)
    xb = synth.token_bf16(8000 + B, B, 512)
    err, y = _parity(L, xb, f"E8M0 extremes B={B} {layout}")
    assert np.all(np.isfinite(y))
