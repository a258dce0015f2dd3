"""GPU matvec parity: moe_expert_gemv_{mxfp4,q2k,int4g32} against the fp64 oracle.

Sizes span several row tiles and a ragged tail (N not a multiple of the
rows per workgroup, K leaving lanes idle), every token count 1..8, and the
full single-matvec workload (W 2048 x 4096 MXFP4, x ~ N(0,1) fp32)."""
import numpy as np
import pytest
import torch

import oracle
import quantized_moe_decode_route_amd as moe
import synth
from gpu_helpers import assert_parity, dev, host

pytestmark = pytest.mark.gpu

SHAPES = [(37, 96), (64, 4096 + 32), (130, 2048), (8, 32)]


def _mx(seed, n, k):
    return synth.mxfp4_blocks(synth.tensor_key(seed, synth.TAG_MXFP4, 0, 0, 0), n * k // 32).reshape(-1)


def _q2(seed, n, k):
    return synth.q2k_blocks(synth.tensor_key(seed, synth.TAG_Q2K, 0, 0, 0), n * k // 256).reshape(-1)


def _run(fmt, w, n, k, x):
    B = x.shape[0]
    y = torch.full((B, n), float("nan"), dtype=torch.float32, device="cuda")
    xd = dev(x.astype(np.float32))
    if fmt == "mxfp4":
        moe.moe_expert_gemv_mxfp4(dev(w), n, k, xd, y)
    elif fmt == "q2k":
        moe.moe_expert_gemv_q2k(dev(w), n, k, xd, y)
    else:
        moe.moe_expert_gemv_int4g32(dev(w[0]), dev(w[1]), n, k, xd, y)
    torch.cuda.synchronize()
    return host(y)


@pytest.mark.parametrize("n,k", SHAPES)
@pytest.mark.parametrize("B", [1, 3, 8])
def test_gemv_mxfp4_parity(n, k, B):
    w = _mx(100 + n, n, k)
    x = synth.token_f32(7 + B, B, k)
    y = _run("mxfp4", w, n, k, x)
    assert_parity(y, oracle.gemv("mxfp4", w, n, k, x.astype(np.float64)), what=f"mxfp4 {n}x{k} B={B}")


@pytest.mark.parametrize("n,k", [(37, 256), (64, 4096), (130, 2048 + 256)])
@pytest.mark.parametrize("B", [1, 2, 8])
def test_gemv_q2k_parity(n, k, B):
    w = _q2(200 + n, n, k)
    x = synth.token_f32(9 + B, B, k)
    y = _run("q2k", w, n, k, x)
    assert_parity(y, oracle.gemv("q2k", w, n, k, x.astype(np.float64)), what=f"q2k {n}x{k} B={B}")


@pytest.mark.parametrize("n,k", SHAPES)
@pytest.mark.parametrize("B", [1, 5, 8])
def test_gemv_int4_parity(n, k, B):
    q, s = synth.int4_raw(synth.tensor_key(300 + n, synth.TAG_INT4, 0, 0, 0), n, k)
    x = synth.token_f32(11 + B, B, k)
    y = _run("int4g32", (q, s), n, k, x)
    assert_parity(y, oracle.gemv("int4g32", (q, s), n, k, x.astype(np.float64)), what=f"int4 {n}x{k} B={B}")


def test_gemv_mxfp4_full_single_matvec_workload():
    # W [2048 x 4096] MXFP4 (uniform codes, E8M0 in 118..134), x ~ N(0,1) fp32, batch 1.
    n, k = 2048, 4096
    w = _mx(0x5EED, n, k)
    x = synth.token_f32(1000, 1, k)
    y = _run("mxfp4", w, n, k, x)
    err = assert_parity(y, oracle.gemv("mxfp4", w, n, k, x.astype(np.float64)), what="cfg0")
    print(f"single matvec 2048x4096: max rel-inf err {err:.3e}")


def test_gemv_every_token_count_and_width_invariance():
    # Token t's result must not depend on how many tokens share the call.
    n, k = 96, 4096
    w = _mx(55, n, k)
    x = synth.token_f32(56, 8, k)
    ref = oracle.gemv("mxfp4", w, n, k, x.astype(np.float64))
    y1 = np.stack([_run("mxfp4", w, n, k, x[t:t + 1])[0] for t in range(8)])
    for B in range(1, 9):
        yb = _run("mxfp4", w, n, k, x[:B])
        assert_parity(yb, ref[:B], what=f"B={B}")
        assert np.array_equal(yb, y1[:B]), f"width drift at B={B}"


@pytest.mark.parametrize("fmt,k", [("mxfp4", 8192 + 32), ("int4g32", 16384), ("q2k", 16384 + 256)])
def test_gemv_long_rows(fmt, k):
    """Rows of more than 256 units (more than the register-held path keeps per
    lane) are streamed, four tokens per pass: parity at every token count that
    mixes four-token passes with single tokens, and each token's result
    bitwise the same whatever B is."""
    n = 21  # three workgroups of 8 rows, the last one ragged
    if fmt == "mxfp4":
        w = _mx(700, n, k)
    elif fmt == "q2k":
        w = _q2(701, n, k)
    else:
        w = synth.int4_raw(synth.tensor_key(702, synth.TAG_INT4, 0, 0, 0), n, k)
    x = synth.token_f32(703, 8, k)
    ref = oracle.gemv(fmt, w, n, k, x.astype(np.float64))
    y8 = _run(fmt, w, n, k, x)
    assert_parity(y8, ref, what=f"{fmt} {n}x{k} B=8")
    for B in (1, 3, 4, 5):
        yb = _run(fmt, w, n, k, x[:B])
        assert_parity(yb, ref[:B], what=f"{fmt} {n}x{k} B={B}")
        assert np.array_equal(yb, y8[:B]), f"{fmt}: width drift at B={B}"


def test_gemv_exact_integer_case():
    # e = 127 and codes {0,2,4,5,6,7} give small integers; with integer x the
    # fp32 sums are exact, so the GPU must equal the oracle exactly.
    n, k = 64, 256
    rng = np.random.default_rng(3)
    blocks = synth.mxfp4_blocks(synth.tensor_key(3, 1, 0, 0, 0), n * k // 32)
    allowed = np.array([0, 2, 4, 5, 6, 7], dtype=np.uint8)
    hi = allowed[rng.integers(0, 6, size=(n * k // 32, 16))]
    lo = allowed[rng.integers(0, 6, size=(n * k // 32, 16))]
    blocks[:, 1:] = (hi << 4) | lo
    blocks[:, 0] = 127
    x = rng.integers(-20, 21, size=(2, k)).astype(np.float32)
    y = _run("mxfp4", blocks.reshape(-1), n, k, x)
    assert np.array_equal(y.astype(np.float64), oracle.gemv("mxfp4", blocks, n, k, x.astype(np.float64)))


def test_gemv_rejects_bad_arguments():
    x = torch.zeros((1, 64), dtype=torch.float32, device="cuda")
    y = torch.zeros((1, 8), dtype=torch.float32, device="cuda")
    w = torch.zeros(8 * 2 * 17, dtype=torch.uint8, device="cuda")
    with pytest.raises(moe.MoeError):
        moe.moe_expert_gemv_mxfp4(w, 8, 48, x, y)      # K % 32
    with pytest.raises(moe.MoeError):
        moe.moe_expert_gemv_q2k(w, 8, 64, x, y)        # K % 256
    x9 = torch.zeros((9, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(moe.MoeError):
        moe.moe_expert_gemv_mxfp4(w, 8, 64, x9, y)     # B > 8


def _with_exponents(blocks, choices, seed):
    b = blocks.reshape(-1, 17).copy()
    b[:, 0] = np.random.default_rng(seed).choice(np.asarray(choices, dtype=np.uint8), size=b.shape[0])
    return b.reshape(-1)


@pytest.mark.parametrize("case", ["low", "high", "mixed"])
@pytest.mark.parametrize("B", [1, 8])
def test_gemv_mxfp4_e8m0_extremes(case, B):
    """Scale bytes at both ends of the E8M0 range: 0 (2^-127, whose fp32 bit
    pattern is subnormal), 1, 2, and 250..254 (up to 2^127), alone or mixed
    with the ordinary 118..134.  x is scaled by a power of two so that every
    result is a finite fp32 number (for the mixed rows the tiny blocks then
    contribute below fp32 resolution)."""
    n, k = 64, 1024
    choices, shift = {"low": ([0, 1, 2], 40), "high": ([250, 251, 252, 253, 254], -40),
                      "mixed": ([0, 1, 2, 120, 127, 134, 250, 254], -110)}[case]
    w = _with_exponents(_mx(61, n, k), choices, 62)
    x = np.ldexp(synth.token_f32(63 + B, B, k).astype(np.float64), shift).astype(np.float32)
    y = _run("mxfp4", w, n, k, x)
    ref = oracle.gemv("mxfp4", w, n, k, x.astype(np.float64))
    assert np.all(np.isfinite(ref)) and np.all(np.abs(ref) < 1e37)
    assert np.all(np.isfinite(y))
    assert_parity(y, ref, what=f"E8M0 {case} B={B}")
