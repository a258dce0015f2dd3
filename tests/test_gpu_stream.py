"""The pure-read probe (moe_stream_read) loads exactly the dwords it claims
to: the XOR of its per-workgroup results equals the XOR of the same dwords
computed on the host, for both load patterns, at sizes that leave ragged
tails (not a multiple of the grid or of the unrolled loop)."""
import numpy as np
import pytest
import torch

import quantized_moe_decode_route_amd as moe
from gpu_helpers import dev, host

pytestmark = pytest.mark.gpu


def _run(buf: np.ndarray, nbytes: int, pattern: str) -> int:
    d = dev(buf)
    sink = torch.zeros(moe.MOE_STREAM_GRID, dtype=torch.int32, device="cuda")
    moe.moe_stream_read(d, nbytes, pattern, sink)
    torch.cuda.synchronize()
    return int(np.bitwise_xor.reduce(host(sink).view(np.uint32)))


@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 48, 2048 * 256 * 16 * 4 + 16 * 777, 37 << 20])
def test_stream_dwordx4_reads_every_dword_once(nbytes):
    rng = np.random.default_rng(nbytes % 1000)
    buf = rng.integers(0, 256, size=nbytes, dtype=np.uint8)
    want = int(np.bitwise_xor.reduce(buf.view(np.uint32)))
    assert _run(buf, nbytes, "dwordx4") == want


@pytest.mark.parametrize("nbytes", [20, 17 * 1000 + 4, 17 * 2048 * 256 * 4 + 17 * 33 + 1, 41 << 20])
def test_stream_mxfp4_reads_each_block_window(nbytes):
    nbytes -= nbytes % 4
    rng = np.random.default_rng(nbytes % 997)
    buf = rng.integers(0, 256, size=nbytes, dtype=np.uint8)
    words = buf.view(np.uint32)
    nb = moe.moe_stream_mxfp4_blocks(nbytes)
    assert nb >= 1 and ((17 * (nb - 1)) & ~3) + 20 <= nbytes
    first = (17 * np.arange(nb, dtype=np.int64)) >> 2          # dword index of each block's window
    want = 0
    for j in range(5):
        want ^= int(np.bitwise_xor.reduce(words[first + j]))
    assert _run(buf, nbytes, "mxfp4") == want


def test_stream_rejects_bad_arguments():
    x = torch.zeros(64, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(moe.MOE_STREAM_GRID, dtype=torch.int32, device="cuda")
    with pytest.raises(moe.MoeError):
        moe.moe_stream_read(x, 40, "dwordx4", sink)        # not a multiple of 16
    with pytest.raises(moe.MoeError):
        moe.moe_stream_read(x, 16, "mxfp4", sink)          # shorter than one block window
