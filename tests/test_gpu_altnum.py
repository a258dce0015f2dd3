"""Alternative numerics of the MXFP4 matvec on the GPU ("ds4.c study notes",
glossary page "quantization": "MXFP4's ROCm native kernel" -- Q8_K
activations with integer dot products -- and "Metal's MXFP4 -> half lookup
table").  Each has its own oracle and tolerance:

* the Q8 quantizer is bit-exact (codes and scales decided in fp32 on both
  sides);
* the integer-dot matvec is compared with the oracle's exact-term sum on the
  same quantized activations, within the fp32 rounding of adding the block
  terms ((blocks + 8) * 2^-24 times the sum of the terms' magnitudes), and
  against the unquantized product within the quantization bound
  sum_k |w_k| * d_k * (1/2 + 127 * 2^-23) plus that rounding;
* the binary16 table is bit-exact; the table matvec is compared with the
  oracle's fp64 sum over the table's values within (K + 64) * 2^-24 *
  sum_k |w_k x_k|."""
import numpy as np
import pytest
import torch

import oracle
import quantized_moe_decode_route_amd as moe
import synth
from gpu_helpers import dev, host

pytestmark = pytest.mark.gpu

SHAPES = [(37, 256), (64, 4096), (130, 2048 + 256), (8, 512)]


def _mx(seed, n, k):
    return synth.mxfp4_blocks(synth.tensor_key(seed, synth.TAG_MXFP4, 0, 0, 0), n * k // 32).reshape(-1)


def _x(seed, B, k):
    # per-256 blocks of different magnitudes, so that the block scales differ
    x = synth.token_f32(seed, B, k).astype(np.float64)
    scale = np.exp2(np.arange(k // 256) % 7 - 3.0)
    return (x * np.repeat(scale, 256)[None, :]).astype(np.float32)


def _quantize(x):
    B, K = x.shape
    q = torch.empty((B, K), dtype=torch.int8, device="cuda")
    d = torch.empty((B, K // 256), dtype=torch.float32, device="cuda")
    moe.moe_q8k_quantize(dev(x), q, d)
    torch.cuda.synchronize()
    return host(q), host(d)


@pytest.mark.parametrize("B,K", [(1, 256), (3, 1024), (8, 4096)])
def test_q8k_quantize_bit_exact(B, K):
    x = _x(40 + B, B, K)
    x[0, :256] = 0.0                               # a block of zeros
    if K >= 512:
        x[0, 256:512] = 0.0
        x[0, 256], x[0, 257:260] = 127.0, [2.5, 3.5, -2.5]  # d = 1: ties to even
    q, d = _quantize(x)
    qo, do = oracle.q8k_quantize(x)
    assert np.array_equal(d.view(np.uint32), do.view(np.uint32))
    assert np.array_equal(q, qo)


@pytest.mark.parametrize("n,k", SHAPES)
@pytest.mark.parametrize("B", [1, 2, 8])
def test_gemv_mxfp4_q8_parity(n, k, B):
    w = _mx(300 + n, n, k)
    x = _x(50 + B, B, k)
    qo, do = oracle.q8k_quantize(x)
    y = torch.full((B, n), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_expert_gemv_mxfp4_q8(dev(w), n, k, dev(qo), dev(do), y)
    torch.cuda.synchronize()
    y = host(y).astype(np.float64)
    yo, absy = oracle.gemv_mxfp4_q8(w, n, k, qo, do)
    tol = (k // 32 + 8) * 2.0 ** -24 * absy + 1e-30
    assert np.all(np.abs(y - yo) <= tol), f"max excess {np.max(np.abs(y - yo) - tol)}"
    # against the unquantized product: the quantization bound
    wabs = np.abs(oracle.dequant("mxfp4", w, n, k))
    dd = np.repeat(do.astype(np.float64), 256, axis=1) * (0.5 + 127 * 2.0 ** -23)
    bound = dd @ wabs.T + tol
    exact = oracle.gemv("mxfp4", w, n, k, x.astype(np.float64))
    assert np.all(np.abs(y - exact) <= bound)
    rel = np.max(np.abs(y - exact)) / np.max(np.abs(exact))
    print(f"q8 path {n}x{k} B={B}: error vs unquantized {rel:.2e} of max|y|")


def test_q8_pipeline_end_to_end_full_shape():
    n, k = 2048, 4096
    w = _mx(333, n, k)
    x = _x(60, 8, k)
    q = torch.empty((8, k), dtype=torch.int8, device="cuda")
    d = torch.empty((8, k // 256), dtype=torch.float32, device="cuda")
    y = torch.empty((8, n), dtype=torch.float32, device="cuda")
    moe.moe_q8k_quantize(dev(x), q, d)
    moe.moe_expert_gemv_mxfp4_q8(dev(w), n, k, q, d, y)
    torch.cuda.synchronize()
    qo, do = oracle.q8k_quantize(x)
    assert np.array_equal(host(q), qo)
    yo, absy = oracle.gemv_mxfp4_q8(w, n, k, qo, do)
    assert np.all(np.abs(host(y).astype(np.float64) - yo) <= (k // 32 + 8) * 2.0 ** -24 * absy + 1e-30)


def test_half_lut_bit_exact():
    lut = torch.zeros((256, 16), dtype=torch.int16, device="cuda")
    moe.moe_mxfp4_half_lut(lut)
    torch.cuda.synchronize()
    assert np.array_equal(host(lut).view(np.uint16), oracle.mxfp4_half_lut())


@pytest.mark.parametrize("n,k", SHAPES + [(2048, 4096)])
@pytest.mark.parametrize("B", [1, 8])
def test_gemv_mxfp4_hlut_parity(n, k, B):
    w = _mx(400 + n, n, k)
    x = synth.token_f32(70 + B, B, k)
    y = torch.full((B, n), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_expert_gemv_mxfp4_hlut(dev(w), n, k, dev(x), y)
    torch.cuda.synchronize()
    y = host(y).astype(np.float64)
    yo = oracle.gemv_mxfp4_half(w, n, k, x.astype(np.float64))
    wabs = np.abs(oracle.dequant("mxfp4", w, n, k))
    tol = (k + 64) * 2.0 ** -24 * (np.abs(x.astype(np.float64)) @ wabs.T)
    assert np.all(np.abs(y - yo) <= tol)
