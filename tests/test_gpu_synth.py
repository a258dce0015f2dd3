"""The GPU fill of the seeded generator writes the same bytes as its host twin."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt,nblocks", [("mxfp4", 262144), ("mxfp4", 37), ("q2k", 32768), ("q2k", 5)])
def test_gpu_fill_matches_host_twin(fmt, nblocks):
    bb = synth.MXFP4_BLOCK_BYTES if fmt == "mxfp4" else synth.Q2K_BLOCK_BYTES
    buf = torch.zeros(nblocks * bb + 64, dtype=torch.uint8, device="cuda")
    synth.gpu_fill(fmt, buf.data_ptr(), 0x5EED, 3, 17, 1, synth.PROJ_UP, nblocks,
                   torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got = host(buf)[: nblocks * bb]
    want = synth.expert_tensor(fmt, 0x5EED, 3, 17, synth.PROJ_UP, *((nblocks, 32) if fmt == "mxfp4"
                                                                     else (nblocks, 256)))
    assert np.array_equal(got, want)
    assert np.all(host(buf)[nblocks * bb:] == 0)


def test_gpu_fill_several_experts_contiguous():
    nb = 2048 * 128
    buf = torch.zeros(3 * nb * 17, dtype=torch.uint8, device="cuda")
    synth.gpu_fill("mxfp4", buf.data_ptr(), 1, 0, 5, 3, synth.PROJ_GATE, nb,
                   torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got = host(buf).reshape(3, -1)
    for j in range(3):
        assert np.array_equal(got[j], synth.expert_tensor("mxfp4", 1, 0, 5 + j, synth.PROJ_GATE, 2048, 4096))
