"""GPU FP4 -> INT4 group-32 conversion: codes and scales bit-exact with the oracle."""
import numpy as np
import pytest
import torch

import oracle
import quantized_moe_decode_route_amd as moe
import synth
from gpu_helpers import dev, host

pytestmark = pytest.mark.gpu


def _convert(mx: np.ndarray, n: int, k: int):
    q = torch.empty((n, k // 8), dtype=torch.int32, device="cuda")
    s = torch.empty((n, k // 32), dtype=torch.int16, device="cuda")
    moe.quantize_fp4_to_int4g32(dev(mx.reshape(-1)), n, k, q, s)
    torch.cuda.synchronize()
    return host(q), host(s, np.uint16)


@pytest.mark.parametrize("n,k", [(1, 32), (7, 96), (2048, 4096), (4096, 2048)])
def test_convert_bit_exact(n, k):
    mx = synth.mxfp4_blocks(synth.tensor_key(40 + n, synth.TAG_MXFP4, 0, 0, 0), n * k // 32)
    q, s = _convert(mx, n, k)
    qo, so = oracle.quantize_fp4_to_int4g32(mx, n, k)
    assert np.array_equal(q, qo)
    assert np.array_equal(s, so)


def test_convert_edge_blocks():
    # all-zero codes (amax clamp, first-candidate tie), all +6 / all -6, a
    # single 6 among halves, the ramp of all 16 codes, every exponent 0..252
    # (e = 0 is the subnormal 2^-127 scale).
    rows = []
    for e in list(range(0, 253, 4)) + [0, 1, 118, 134, 252]:
        for codes in ([0] * 32, [7] * 32, [15] * 32, [7] + [1] * 31, list(range(16)) * 2, [8] * 32):
            qs = [(codes[2 * j] << 4) | codes[2 * j + 1] for j in range(16)]
            rows.append([e] + qs)
    mx = np.array(rows, dtype=np.uint8)
    n = mx.shape[0]
    q, s = _convert(mx, n, 32)
    qo, so = oracle.quantize_fp4_to_int4g32(mx, n, 32)
    bad = np.nonzero((q != qo).any(axis=1) | (s[:, 0] != so[:, 0]))[0]
    assert bad.size == 0, f"mismatch in rows {bad[:10]} (exponents {mx[bad[:10], 0]})"


def test_convert_random_exponents_full_range():
    rng = np.random.default_rng(5)
    mx = rng.integers(0, 256, size=(50000, 17), dtype=np.uint8)
    mx[:, 0] = rng.integers(0, 253, size=50000)
    q, s = _convert(mx, 50000, 32)
    qo, so = oracle.quantize_fp4_to_int4g32(mx, 50000, 32)
    assert np.array_equal(q, qo) and np.array_equal(s, so)


def test_validate_counts_infinite_scales():
    mx = synth.mxfp4_blocks(synth.tensor_key(9, synth.TAG_MXFP4, 0, 0, 0), 1000)
    mx[[3, 500, 999], 0] = 0xFF
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    moe.moe_validate_mxfp4(dev(mx.reshape(-1)), 1000, bad)
    torch.cuda.synchronize()
    assert int(bad.item()) == 3
