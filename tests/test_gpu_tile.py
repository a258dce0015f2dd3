"""GPU block permutations to the 256-column tiled layout (moe_tile_weights)
and to its matrix-core refinement (moe_tile_weights_mfma16): bit-exact
against the same permutations written with numpy reshapes.

Inputs are the seeded generators' blocks (MXFP4, Q2_K) and seeded random INT4
words and scales; the expected bytes never come from the HIP path."""
import numpy as np
import pytest
import torch

import quantized_moe_decode_route_amd as moe
import synth
from gpu_helpers import dev, host

pytestmark = pytest.mark.gpu


def _tiled(a: np.ndarray, n: int, tiles: int) -> np.ndarray:
    """Row-major [n][tiles * w] -> tile-major [tiles][n][w] (w = elements of one tile row)."""
    return np.ascontiguousarray(a.reshape(n, tiles, -1).transpose(1, 0, 2)).reshape(-1)


@pytest.mark.parametrize("fmt", ["mxfp4", "q2k"])
@pytest.mark.parametrize("n,k", [(1, 256), (37, 512), (4096, 2048)])
def test_tile_blocks_bit_exact(fmt, n, k):
    bw, bb = (32, 17) if fmt == "mxfp4" else (256, 84)
    key = synth.tensor_key(90 + n, synth.TAG_MXFP4 if fmt == "mxfp4" else synth.TAG_Q2K, 0, 0, 2)
    blocks = synth.mxfp4_blocks(key, n * k // bw) if fmt == "mxfp4" else synth.q2k_blocks(key, n * k // bw)
    src = dev(blocks.reshape(-1))
    dst = torch.empty_like(src)
    moe.moe_tile_weights(fmt, src, n, k, dst)
    torch.cuda.synchronize()
    assert np.array_equal(host(dst), _tiled(blocks.reshape(-1), n, k // 256))


@pytest.mark.parametrize("n,k", [(3, 256), (130, 768), (4096, 2048)])
def test_tile_int4_codes_and_scales_bit_exact(n, k):
    rng = np.random.default_rng(1234 + n)
    q = rng.integers(-2**31, 2**31, size=(n, k // 8), dtype=np.int64).astype(np.int32)
    s = rng.integers(0, 2**16, size=(n, k // 32), dtype=np.int64).astype(np.uint16)
    qd, sd = dev(q.reshape(-1)), dev(s.reshape(-1))
    qt, st = torch.empty_like(qd), torch.empty_like(sd)
    moe.moe_tile_weights("int4g32", qd, n, k, qt, src_scale=sd, dst_scale=st)
    torch.cuda.synchronize()
    assert np.array_equal(host(qt), _tiled(q.reshape(-1), n, k // 256))
    assert np.array_equal(host(st, np.uint16), _tiled(s.reshape(-1), n, k // 256))


def _mfma16(blocks: np.ndarray, n: int, k: int) -> np.ndarray:
    """[n][k/32] blocks -> [tile c][row group n/16][half][quarter][row n%16] (MOE_LAYOUT_MFMA16)."""
    b = blocks.reshape(n // 16, 16, k // 256, 2, 4, 17)          # (R, i, c, h, q, byte)
    return np.ascontiguousarray(b.transpose(2, 0, 3, 4, 1, 5)).reshape(-1)


@pytest.mark.parametrize("n,k", [(16, 256), (48, 768), (4096, 2048)])
def test_tile_mfma16_bit_exact(n, k):
    key = synth.tensor_key(190 + n, synth.TAG_MXFP4, 0, 0, 2)
    blocks = synth.mxfp4_blocks(key, n * k // 32)
    src = dev(blocks.reshape(-1))
    dst = torch.empty_like(src)
    moe.moe_tile_weights_mfma16(src, n, k, dst)
    torch.cuda.synchronize()
    assert np.array_equal(host(dst), _mfma16(blocks.reshape(-1), n, k))
