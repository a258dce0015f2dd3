"""Width exactness of the verify path: a token's result must not depend on how
many other tokens share the call ([mixed] "Width drift" and "Why this is not a
host-side patch": a speculative-verify batch of K+1 tokens must reproduce the
one-token decode bit for bit).

For every batch width B = 1..8, every weight format and down layout, both
launch paths (the single-launch kernel and the multi-launch fallback) and the
layer stack, the B-token call's row t equals the one-token call of token t,
bit for bit, and so do the routing decisions.  Results also reproduce after
the workspace is re-initialised and in a fresh process."""
import hashlib
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import quantized_moe_decode_route_amd as moe
import synth
from gpu_helpers import Layer, dev, host

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _widths(L, x8):
    """Rows of the one-token calls, then of every wider call, compared."""
    ws = L.workspace(8)
    ones = [L.run(x8[t:t + 1], ws) for t in range(8)]
    for B in range(2, 9):
        y, idx, gw = L.run(x8[:B], ws)
        for t in range(B):
            assert np.array_equal(idx[t], ones[t][1][0]), f"B={B} token {t}: routing differs from B=1"
            assert np.array_equal(gw[t].view(np.uint32), ones[t][2][0].view(np.uint32)), f"B={B} token {t}: weights"
            assert np.array_equal(y[t].view(np.uint32), ones[t][0][0].view(np.uint32)), \
                f"B={B} token {t}: row differs from the one-token call"
    return ones


@pytest.mark.parametrize("fmt,layout", [(f, l) for f in ("mxfp4", "q2k", "int4g32") for l in ("rows", "tile256")]
                         + [("mxfp4", "mfma16")])
def test_every_width_small(fmt, layout):
    L = Layer(fmt, 0x77, 0, 32, 512, 256, 6, down_layout=layout)
    _widths(L, synth.token_bf16(8100, 8, 512))


@pytest.mark.parametrize("layout", ["rows", "mfma16"])
def test_every_width_multi_launch_fallback(layout):
    # d_model 8192: runs as separate launches (route, gate/up, down, combine)
    L = Layer("mxfp4", 0x78, 0, 16, 8192, 512, 6, down_layout=layout)
    _widths(L, synth.token_bf16(8200, 8, 8192))


@pytest.mark.parametrize("fmt,layout", [("mxfp4", "mfma16"), ("q2k", "tile256"), ("int4g32", "tile256")])
def test_every_width_full_shape(fmt, layout):
    L = Layer(fmt, 0x79, 0, 256, 4096, 2048, 6, down_layout=layout)
    _widths(L, synth.token_bf16(8300, 8, 4096))
    del L
    torch.cuda.empty_cache()


def test_every_width_stack():
    """Three stacked MXFP4 layers: the one-token step normalises inside the
    layer kernel, wider steps use the norm kernel; the rows still agree."""
    E, D, F = 32, 512, 256
    layers = [Layer("mxfp4", 0x7A, l, E, D, F, 6, down_layout="mfma16") for l in range(3)]
    descs = [L.desc for L in layers]
    h8 = synth.f32_from_bf16_bits(synth.token_bf16(8400, 8, D)) * np.float32(2.0)
    ws = torch.empty(moe.moe_stack_workspace_bytes(8, D, F, E, 6), dtype=torch.uint8, device="cuda")
    moe.moe_workspace_init(ws)

    def stack(h):
        hin = dev(h)
        hout = torch.empty_like(hin)
        moe.moe_stack_decode(descs, hin, hout, ws)
        torch.cuda.synchronize()
        return host(hout)

    ones = [stack(h8[t:t + 1])[0] for t in range(8)]
    for B in range(2, 9):
        out = stack(h8[:B])
        for t in range(B):
            assert np.array_equal(out[t].view(np.uint32), ones[t].view(np.uint32)), f"stack B={B} token {t}"


_REPRO = r"""
import sys, hashlib
sys.path.insert(0, {root!r}); sys.path.insert(0, {root!r} + "/tests")
import numpy as np, torch
import synth
from gpu_helpers import Layer
L = Layer("mxfp4", 0x7B, 0, 32, 512, 256, 6, down_layout="mfma16")
h = hashlib.sha256()
for B in (1, 5, 8):
    y, idx, gw = L.run(synth.token_bf16(8500 + B, B, 512))
    h.update(y.tobytes()); h.update(idx.tobytes()); h.update(gw.tobytes())
print(h.hexdigest())
"""


def _digest(L):
    h = hashlib.sha256()
    for B in (1, 5, 8):
        y, idx, gw = L.run(synth.token_bf16(8500 + B, B, 512))
        h.update(y.tobytes())
        h.update(idx.tobytes())
        h.update(gw.tobytes())
    return h.hexdigest()


def test_reproduces_after_reinit_and_in_a_fresh_process():
    L = Layer("mxfp4", 0x7B, 0, 32, 512, 256, 6, down_layout="mfma16")
    first = _digest(L)            # each run() makes and initialises a fresh workspace
    assert _digest(L) == first
    out = subprocess.run([sys.executable, "-c", _REPRO.format(root=ROOT)], capture_output=True, text=True,
                         timeout=300)
    assert out.returncode == 0, out.stderr[-2000:]
    assert out.stdout.strip().splitlines()[-1] == first, "a fresh process gave different bits"
