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


def _midpoint_rows(rng, B, D):
    """Rows of 3 * (a bfloat16 value or a bfloat16 rounding midpoint in
    [0.5, 1)), random signs: every h^2 has at most 22 significant bits, so
    mean(h^2) is exact in any summation order and eps = 9 - mean makes the
    divisor exactly 3: each quotient is then exactly a bfloat16 value or a
    midpoint (a tie, rounded to even).  The odd rows move every element one
    fp32 step (up or toward zero), which puts the quotients a fraction of an
    fp32 step beside the midpoints."""
    b = rng.integers(0x3F00, 0x3F80, size=(B, D)).astype(np.uint32)
    half = np.where(rng.random((B, D)) < 0.75, 0x8000, 0).astype(np.uint32)
    m = ((b << 16) | half).view(np.float32).astype(np.float64)
    sign = np.where(rng.random((B, D)) < 0.5, -1.0, 1.0)
    h = (3.0 * m * sign).astype(np.float32)
    up = rng.random((B, D)) < 0.5
    moved = np.where(up, np.nextafter(h, np.float32(np.inf)), np.nextafter(h, np.float32(0)))
    h[1::2] = moved[1::2]
    return h


@pytest.mark.parametrize("D", [4096, 8192])
def test_rmsnorm_midpoints_and_subnormals(D):
    """The fast fp32 quotient must fall back to the exact fp64 one wherever it
    could round differently: exact midpoints (ties to even), neighbours of
    midpoints, quotients in the fp32 subnormal range and divisors whose
    reciprocal is not a normal fp32 number.  D = 4096 takes the one-chunk-
    per-thread path, D = 8192 the element walk."""
    rng = np.random.default_rng(5)
    h = _midpoint_rows(rng, 4, D)
    for t in range(4):
        mean = float(np.sum(h[t].astype(np.float64) ** 2) / D)
        eps = max(9.0 - mean, 0.0)
        if t % 2 == 0:
            assert mean + eps == 9.0
        x = torch.empty((1, D), dtype=torch.int16, device="cuda")
        moe.moe_rmsnorm_bf16(dev(h[t:t + 1]), x, float(eps))
        torch.cuda.synchronize()
        want = oracle.rmsnorm_bf16(h[t:t + 1].astype(np.float64), float(eps))
        assert np.array_equal(host(x, np.uint16), want), f"row {t}"
    # subnormal quotients beside one large element; all-subnormal rows (1/denom
    # beyond fp32); a zero row with eps > 0
    tiny = (rng.standard_normal((3, D)) * 1e-42).astype(np.float32)
    tiny[0, 17] = 1e3
    tiny[2] = 0.0
    x = torch.empty((3, D), dtype=torch.int16, device="cuda")
    moe.moe_rmsnorm_bf16(dev(tiny), x, 1e-6)
    torch.cuda.synchronize()
    assert np.array_equal(host(x, np.uint16)[:2], oracle.rmsnorm_bf16(tiny[:2].astype(np.float64), 1e-6)[:2])
    got0 = host(x, np.uint16)[2]
    assert np.all(got0 == 0)
    x1 = torch.empty((1, D), dtype=torch.int16, device="cuda")
    moe.moe_rmsnorm_bf16(dev(tiny[1:2]), x1, 0.0)
    torch.cuda.synchronize()
    assert np.array_equal(host(x1, np.uint16), oracle.rmsnorm_bf16(tiny[1:2].astype(np.float64), 0.0))


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


@pytest.mark.parametrize("fmt,layout,B,D,F,E", [
    ("mxfp4", "mfma16", 1, 512, 256, 32), ("mxfp4", "mfma16", 1, 4096, 2048, 256),
    ("mxfp4", "mfma16", 1, 992, 256, 32), ("mxfp4", "rows", 1, 512, 256, 32),
    ("q2k", "rows", 8, 512, 256, 32), ("mxfp4", "mfma16", 8, 4096, 2048, 256)])
def test_stack_in_kernel_norm_matches_norm_kernel(fmt, layout, B, D, F, E):
    """A one-token stack step with the MXFP4 matrix-core layer normalises its
    input inside the single-launch layer kernel; run in place (h_out aliasing
    h_in) with one layer, the separate norm kernel does it instead.  Both
    define the same sum order and the same rounding, so the residual states
    agree bit for bit.  (The other cases take the norm kernel both ways.)"""
    layers = [Layer(fmt, 0x5EED + 40 + B, l, E, D, F, 6, down_layout=layout) for l in range(2)]
    h = synth.f32_from_bf16_bits(synth.token_bf16(4100 + B, B, D)) * np.float32(3.0)
    ws = torch.empty(moe.moe_stack_workspace_bytes(B, D, F, E, 6), dtype=torch.uint8, device="cuda")
    moe.moe_workspace_init(ws)
    for l in range(2):
        hin = dev(h)
        hout = torch.empty_like(hin)
        moe.moe_stack_decode([layers[l].desc], hin, hout, ws)       # in-kernel norm
        inplace = dev(h)
        moe.moe_stack_decode([layers[l].desc], inplace, inplace, ws)  # norm kernel, then the layer
        torch.cuda.synchronize()
        a, b = host(hout), host(inplace)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"layer {l}"
        h = a
    # two layers in one call (each normalising in-kernel) give the same bits
    hin = dev(synth.f32_from_bf16_bits(synth.token_bf16(4100 + B, B, D)) * np.float32(3.0))
    hout = torch.empty_like(hin)
    moe.moe_stack_decode([L.desc for L in layers], hin, hout, ws)
    torch.cuda.synchronize()
    assert np.array_equal(host(hout).view(np.uint32), h.view(np.uint32))
    del layers
    torch.cuda.empty_cache()


@pytest.mark.parametrize("B,layout", [(1, "rows"), (1, "mfma16"), (8, "mfma16")])
def test_stack_full_shape_three_layers(B, layout):
    """Three full-shape layers (256 experts, 4096 x 2048), checked layer by
    layer with teacher forcing.  At B = 8 with the matrix-core layout the norm
    kernel feeds the layer and the residual is added in the layer's finish;
    at B = 1 with that layout the layer normalises its input itself."""
    D, F, E = 4096, 2048, 256
    layers = [Layer("mxfp4", 0x5EED + 4, l, E, D, F, 6, down_layout=layout) for l in range(3)]
    x0 = synth.token_bf16(4000 + B, B, D)
    h0 = synth.f32_from_bf16_bits(x0)
    ws = torch.empty(moe.moe_stack_workspace_bytes(B, D, F, E, 6), dtype=torch.uint8, device="cuda")
    moe.moe_workspace_init(ws)
    hs = [h0]
    for l in range(3):
        hin = dev(hs[-1])
        hout = torch.empty_like(hin)
        moe.moe_stack_decode([layers[l].desc], hin, hout, ws)
        torch.cuda.synchronize()
        hs.append(host(hout))
    assert moe.moe_workspace_flags(ws) == 0
    for l in range(3):
        xl = oracle.rmsnorm_bf16(hs[l].astype(np.float64))
        y, _, _ = layers[l].oracle(xl)
        err = assert_parity(hs[l + 1].astype(np.float64) - hs[l].astype(np.float64), y,
                            what=f"full layer {l} B={B} {layout}")
        print(f"stack full shape B={B} {layout} layer {l}: max rel-inf err {err:.3e}")
    # the three layers in one call give the same bits
    hin = dev(h0)
    hout = torch.empty_like(hin)
    moe.moe_stack_decode([L.desc for L in layers], hin, hout, ws)
    torch.cuda.synchronize()
    assert np.array_equal(host(hout).view(np.uint32), hs[-1].view(np.uint32))
    del layers
    torch.cuda.empty_cache()


@pytest.mark.parametrize("B", [1, 8])
def test_stack_free_running_against_oracle_stack(B):
    """Two layers in one call against oracle.stack_decode, which runs the
    same residual recursion in fp64 from the same fp32 state.

    Free running, the GPU's fp32 residual after layer 0 differs from the
    oracle's fp64 one at fp32 resolution, and the bfloat16 rounding of the
    norm can turn that into a one-unit difference of an element of x_1 (the
    next layer then sees a different input: ~2^-8 of that element).  So a
    token is held to the 1e-4 bar against the oracle's stack where its x_1
    is the oracle's bit for bit; elsewhere x_1 may differ by about one
    bfloat16 unit (more for elements far below the largest, whose absolute error is
    set by the largest), and that layer is checked with teacher forcing (the
    GPU's own x_1 through the oracle layer)."""
    E, D, F = 32, 512, 256
    layers = [Layer("mxfp4", 0x5EED + 90, l, E, D, F, 6, down_layout="mfma16") for l in range(2)]
    h0 = synth.token_f32(4200 + B, B, D) * np.float32(2.0)
    ws = torch.empty(moe.moe_stack_workspace_bytes(B, D, F, E, 6), dtype=torch.uint8, device="cuda")
    moe.moe_workspace_init(ws)
    hin = dev(h0)
    hout = torch.empty_like(hin)
    moe.moe_stack_decode([L.desc for L in layers], hin, hout, ws)
    h1 = torch.empty_like(hin)
    moe.moe_stack_decode([layers[0].desc], hin, h1, ws)
    torch.cuda.synchronize()
    h2, h1 = host(hout), host(h1)
    href, steps = oracle.stack_decode("mxfp4", lambda l, e: layers[l].expert_host(e), [L.router for L in layers],
                                      h0, 6, F, trace=True)
    assert_parity(h1, h0.astype(np.float64) + steps[0][3], what=f"stack layer 0 B={B}")
    x1 = oracle.rmsnorm_bf16(h1.astype(np.float64))
    same = np.all(x1 == steps[1][0], axis=1)
    if same.any():
        assert_parity(h2[same], href[same], what=f"two-layer stack B={B}")
    if not same.all():
        up = oracle.bf16_rows_to_f64(x1[~same])
        ref = oracle.bf16_rows_to_f64(steps[1][0][~same])
        # layer 0 holds |dh| <= 1e-4 ||h||_inf, i.e. |dx| <= 1e-4 max|x| after
        # the norm, and the bfloat16 rounding adds at most one unit
        ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(up), np.abs(ref)))[1] - 8)
        assert np.all(np.abs(up - ref) <= ulp + 2e-4 * np.max(np.abs(ref), axis=1, keepdims=True))
        y1, _, _ = layers[1].oracle(x1[~same])
        assert_parity(h2[~same].astype(np.float64) - h1[~same].astype(np.float64), y1,
                      what=f"two-layer stack B={B}, layer 1 teacher-forced")
