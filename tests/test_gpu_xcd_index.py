"""A workgroup's index inside its XCD decides which d_ff rows and output rows
it owns.  When the placement probe saw workgroup b run on XCD b % XCDs the
library takes the index from the block index (blockIdx / XCDs); with
MOE_XCD_INDEX_ATOMIC set, or any other placement, it takes it from an L2
atomic counter.  The ownership changes nothing in a row's arithmetic, so both
ways give the same bits: checked at the full layer shape (256 experts,
4096 x 2048) for the matrix-core MXFP4 path, Q2_K and INT4, at one and eight
tokens, against a child process that uses the counter."""
import ctypes
import hashlib
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import quantized_moe_decode_route_amd as moe
import synth
from gpu_helpers import Layer

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_CASES = (("mxfp4", "mfma16"), ("q2k", "tile256"), ("int4g32", "tile256"))

_CHILD = r"""
import ctypes, hashlib, sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import numpy as np, torch
import synth
import quantized_moe_decode_route_amd as moe
from gpu_helpers import Layer
{index_field}
for fmt, layout in {cases!r}:
    L = Layer(fmt, 0x1DC, 0, 256, 4096, 2048, 6, down_layout=layout)
    h = hashlib.sha256()
    for B in (1, 8):
        y, idx, gw = L.run(synth.token_bf16(8700 + B, B, 4096))
        h.update(y.tobytes()); h.update(idx.tobytes()); h.update(gw.tobytes())
    print(fmt, h.hexdigest())
    if fmt == "mxfp4":
        print("index_field", int((index_field(L)[0] >> np.uint64(63)).max()))
    del L
"""

_INDEX_FIELD = r"""
def index_field(L):
    x = torch.from_numpy(synth.token_bf16(8800, 1, 4096).view(np.int16)).to("cuda")
    y = torch.empty((1, 4096), dtype=torch.float32, device="cuda")
    ws = L.workspace(1)
    nb = ctypes.c_int(0)
    lib = moe.lib()
    args = (ctypes.byref(L.desc), x.data_ptr(), 1, y.data_ptr(), ws.data_ptr(), ws.numel())
    assert lib.moe_layer_decode_traced(*args, None, ctypes.byref(nb), None) == 0
    tr = torch.zeros((nb.value, moe.TRACE_FIELDS), dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    assert lib.moe_layer_decode_traced(*args, tr.data_ptr(), ctypes.byref(nb), stream) == 0
    torch.cuda.synchronize()
    t = tr.cpu().numpy().view(np.uint64)
    return t[:, moe.TRACE_FIELDS - 1], t[:, moe.TRACE_FIELDS - 2]
"""
exec(_INDEX_FIELD)


def _digests():
    out = {}
    for fmt, layout in _CASES:
        L = Layer(fmt, 0x1DC, 0, 256, 4096, 2048, 6, down_layout=layout)
        if fmt == "mxfp4":
            field, xcd = index_field(L)
            # every workgroup took its index from the block index, and the indices
            # on each XCD are 0 .. grid/NX - 1 once each
            assert ((field >> np.uint64(63)) == 1).all(), "the block-index mode is not in use"
            idx = (field & np.uint64(0xFFFFFFFF)).astype(np.int64)
            for x in np.unique(xcd):
                got = np.sort(idx[xcd == x])
                assert np.array_equal(got, np.arange(len(got))), f"XCD {x}: indices {got}"
        h = hashlib.sha256()
        for B in (1, 8):
            y, idx, gw = L.run(synth.token_bf16(8700 + B, B, 4096))
            h.update(y.tobytes())
            h.update(idx.tobytes())
            h.update(gw.tobytes())
        out[fmt] = h.hexdigest()
        del L
    return out


def test_cu_position_index_equals_atomic_index():
    here = _digests()
    env = dict(os.environ, MOE_XCD_INDEX_ATOMIC="1")
    code = _CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), cases=_CASES, index_field=_INDEX_FIELD)
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600, env=env)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [line.split() for line in res.stdout.strip().splitlines() if line.strip()]
    child = {w[0]: w[1] for w in lines if w[0] in here}
    assert ["index_field", "0"] in lines, "the child did not use the arrival counter"
    for fmt in here:
        assert child[fmt] == here[fmt], f"{fmt}: the counter-indexed layer gave different bits"
