"""Error distribution of the fp32-accumulated layer outputs against the fp64
oracle, over many tokens at the full layer shape (256 experts, 4096 x 2048,
MXFP4) for the down-projection layouts side by side: the matrix-core path
(MOE_LAYOUT_MFMA16: h as E4M3 terms in the scaled MFMA) and the vector path
(MOE_LAYOUT_TILE256).  Each token's error is max |y_gpu - y_oracle| /
max |y_oracle|; the bar is 1e-4.  The distribution is printed (run with -s)."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import Layer, rel_inf_err

pytestmark = pytest.mark.gpu

N_TOK = 64


def _dist(errs):
    e = np.asarray(errs)
    q = np.percentile(e, [50, 90, 99])
    return f"max {e.max():.3e}  p99 {q[2]:.3e}  p90 {q[1]:.3e}  p50 {q[0]:.3e}  mean {e.mean():.3e}"


@pytest.mark.parametrize("shape", ["full", "small"])
@pytest.mark.parametrize("layout", ["mfma16", "tile256"])
@pytest.mark.parametrize("B", [1, 8])
def test_error_distribution(shape, layout, B):
    E, D, F = (256, 4096, 2048) if shape == "full" else (16, 512, 256)
    L = Layer("mxfp4", 0x5EED + 100, 0, E, D, F, 6, down_layout=layout)
    errs = []
    ws = L.workspace(B)
    for i in range(N_TOK // B):
        xb = synth.token_bf16(9000 + i, B, D)
        y, idx, _ = L.run(xb, ws)
        yo, io, _ = L.oracle(xb)
        assert np.array_equal(idx, io)
        errs.extend(rel_inf_err(y, yo).tolist())
    print(f"\n{shape} {layout} B={B} ({len(errs)} tokens): {_dist(errs)}")
    assert max(errs) <= 1e-4
    del L
    torch.cuda.empty_cache()


@pytest.mark.parametrize("shape", ["full", "small"])
@pytest.mark.parametrize("fmt", ["int4g32", "q2k"])
@pytest.mark.parametrize("B", [1, 8])
def test_error_distribution_vector_formats(shape, fmt, B):
    """The same distribution for the formats whose down projection runs on the
    vector path (256-column tiled down): INT4 group-32, whose down dot takes h
    as six planes of base-16 digits against the stored codes, and Q2_K."""
    E, D, F = (256, 4096, 2048) if shape == "full" else (16, 512, 256)
    L = Layer(fmt, 0x5EED + 200, 0, E, D, F, 6, down_layout="tile256")
    errs = []
    ws = L.workspace(B)
    for i in range(32 // B):
        xb = synth.token_bf16(9500 + i, B, D)
        y, idx, _ = L.run(xb, ws)
        yo, io, _ = L.oracle(xb)
        assert np.array_equal(idx, io)
        errs.extend(rel_inf_err(y, yo).tolist())
    print(f"\n{shape} {fmt} tile256 B={B} ({len(errs)} tokens): {_dist(errs)}")
    assert max(errs) <= 1e-4
    del L
    torch.cuda.empty_cache()
