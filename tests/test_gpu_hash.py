"""Hash-routed layers on the GPU ("cabbage v4x quant surgery": the first 3 of
the 43 layers map each token to experts by a fixed hash of its id, the
tid2eid table, instead of by the learned router).  The table here is a
seeded stand-in (the pages do not give the hash function).  Parity against
the oracle on both launch paths and at every batch width, the invalid-input
rule (a bad id or row routes the token to experts 0..k-1 and raises the
workspace flag), and a stack whose first layer is hash-routed."""
import numpy as np
import pytest
import torch

import oracle
import quantized_moe_decode_route_amd as moe
import synth
from gpu_helpers import Layer, assert_parity, dev, host

pytestmark = pytest.mark.gpu

VOCAB = 1000


class Hashed:
    """A Layer made hash-routed: its descriptor gains a device tid2eid table."""

    def __init__(self, L: Layer, seed: int):
        self.L = L
        self.table = synth.tid2eid_table(seed, VOCAB, L.E, L.k)
        self.table_dev = dev(self.table)
        self.desc = moe.moe_layer_desc.from_buffer_copy(L.desc)
        self.desc.tid2eid, self.desc.vocab = self.table_dev.data_ptr(), VOCAB

    def run(self, ids, xb, ws=None):
        L = self.L
        B = xb.shape[0]
        ws = ws if ws is not None else L.workspace(B)
        y = torch.empty((B, L.D), dtype=torch.float32, device="cuda")
        idx = torch.empty((B, L.k), dtype=torch.int32, device="cuda")
        gw = torch.empty((B, L.k), dtype=torch.float32, device="cuda")
        moe.moe_layer_decode_ids(self.desc, dev(ids), dev(xb), y, ws, idx, gw)
        torch.cuda.synchronize()
        return host(y), host(idx), host(gw), moe.moe_workspace_flags(ws)

    def oracle(self, ids, xb):
        L = self.L
        return oracle.layer_decode((L.fmt, L.down_fmt), L.expert_host, L.router, xb, L.k, L.F,
                                   hashed=(self.table, ids))


def _parity(H, ids, xb, what):
    y, idx, gw, flags = H.run(ids, xb)
    yo, io, go = H.oracle(ids, xb)
    assert flags == 0, f"{what}: flags {flags}"
    assert np.array_equal(idx, io), f"{what}: experts differ"
    assert np.array_equal(idx, H.table[ids]), f"{what}: not the table's experts"
    assert np.max(np.abs(gw - go)) <= 1e-6
    return assert_parity(y, yo, what=what)


@pytest.mark.parametrize("layout", ["rows", "mfma16"])
def test_hashed_small(layout):
    H = Hashed(Layer("mxfp4", 0xA1, 0, 32, 512, 256, 6, down_layout=layout), 0xA1)
    for B in (1, 3, 8):
        _parity(H, synth.token_ids(100 + B, B, VOCAB), synth.token_bf16(10100 + B, B, 512), f"hashed B={B}")


def test_hashed_other_formats():
    H = Hashed(Layer("int4g32", 0xA2, 0, 32, 512, 512, 6, down_layout="tile256", down_fmt="q2k"), 0xA2)
    for B in (1, 8):
        _parity(H, synth.token_ids(200 + B, B, VOCAB), synth.token_bf16(10200 + B, B, 512), f"int4+q2k B={B}")


def test_hashed_multi_launch_fallback():
    H = Hashed(Layer("mxfp4", 0xA3, 0, 16, 8192, 512, 6), 0xA3)
    for B in (1, 8):
        _parity(H, synth.token_ids(300 + B, B, VOCAB), synth.token_bf16(10300 + B, B, 8192), f"fallback B={B}")


@pytest.mark.parametrize("B", [1, 8])
def test_hashed_full_shape(B):
    H = Hashed(Layer("mxfp4", 0xA4, 0, 256, 4096, 2048, 6, down_layout="mfma16"), 0xA4)
    err = _parity(H, synth.token_ids(400 + B, B, VOCAB), synth.token_bf16(10400 + B, B, 4096), f"full B={B}")
    print(f"hashed mxfp4 layer B={B}: max rel-inf err {err:.3e}")
    del H
    torch.cuda.empty_cache()


def test_hashed_every_width():
    H = Hashed(Layer("mxfp4", 0xA5, 0, 32, 512, 256, 6, down_layout="mfma16"), 0xA5)
    ids8, x8 = synth.token_ids(500, 8, VOCAB), synth.token_bf16(10500, 8, 512)
    ws = H.L.workspace(8)
    ones = [H.run(ids8[t:t + 1], x8[t:t + 1], ws) for t in range(8)]
    for B in range(2, 9):
        y, idx, _, _ = H.run(ids8[:B], x8[:B], ws)
        for t in range(B):
            assert np.array_equal(idx[t], ones[t][1][0])
            assert np.array_equal(y[t].view(np.uint32), ones[t][0][0].view(np.uint32)), f"B={B} token {t}"


@pytest.mark.parametrize("shape", [(32, 512, 256), (16, 8192, 512)])
def test_hashed_invalid_ids_and_rows(shape):
    """Out-of-range ids, experts outside [0, E) and repeated experts: those
    tokens use experts 0..k-1 (as the oracle does), the flag is raised, and
    re-initialising the workspace clears it."""
    E, D, F = shape
    H = Hashed(Layer("mxfp4", 0xA6, 0, E, D, F, 6), 0xA6)
    H.table[3, 2] = H.table[3, 4]          # a repeated expert
    H.table[5, 0] = E                      # an expert past the last
    H.table[6, 1] = -1
    H.table_dev.copy_(dev(H.table))
    ids = np.array([3, 5, 6, VOCAB, -2, 9], dtype=np.int32)
    xb = synth.token_bf16(10600, 6, D)
    ws = H.L.workspace(8)
    y, idx, gw, flags = H.run(ids, xb, ws)
    yo, io, go = H.oracle(ids, xb)
    assert flags & 2, "bad-input flag not raised"
    assert np.array_equal(idx, io)
    assert all(idx[t].tolist() == list(range(6)) for t in range(5)) and np.array_equal(idx[5], H.table[9])
    assert_parity(y, yo, what="invalid rows")
    moe.moe_workspace_init(ws)
    torch.cuda.synchronize()
    assert moe.moe_workspace_flags(ws) == 0
    _, _, _, flags = H.run(np.array([1, 2], dtype=np.int32), xb[:2], ws)
    assert flags == 0


@pytest.mark.parametrize("B", [1, 8])
def test_stack_with_hashed_first_layer(B):
    """Like the model's first layers: layer 0 hash-routed, then learned layers;
    layer-by-layer parity against the oracle fed the GPU's residual state, and
    the whole stack in one call gives the same bits."""
    E, D, F = 32, 512, 256
    layers = [Layer("mxfp4", 0xA7, l, E, D, F, 6, down_layout="mfma16") for l in range(3)]
    H = Hashed(layers[0], 0xA7)
    descs = [H.desc] + [L.desc for L in layers[1:]]
    ids = synth.token_ids(700 + B, B, VOCAB)
    ids_dev = dev(ids)
    h0 = synth.f32_from_bf16_bits(synth.token_bf16(10700 + B, B, D))
    ws = torch.empty(moe.moe_stack_workspace_bytes(B, D, F, E, 6), dtype=torch.uint8, device="cuda")
    moe.moe_workspace_init(ws)
    hs = [h0]
    for l in range(3):
        hin = dev(hs[-1])
        hout = torch.empty_like(hin)
        moe.moe_stack_decode_ids([descs[l]], ids_dev, hin, hout, ws)
        torch.cuda.synchronize()
        hs.append(host(hout))
    for l in range(3):
        xl = oracle.rmsnorm_bf16(hs[l].astype(np.float64))
        if l == 0:
            y, idx, _ = H.oracle(ids, xl)
            assert np.array_equal(idx, H.table[ids])
        else:
            y, _, _ = layers[l].oracle(xl)
        assert_parity(hs[l + 1].astype(np.float64) - hs[l].astype(np.float64), y, what=f"layer {l}")
    hin = dev(h0)
    hout = torch.empty_like(hin)
    moe.moe_stack_decode_ids(descs, ids_dev, hin, hout, ws)
    torch.cuda.synchronize()
    assert np.array_equal(host(hout), hs[-1])
    assert moe.moe_workspace_flags(ws) == 0
    with pytest.raises(RuntimeError):
        moe.moe_stack_decode(descs, hin, hout, ws)        # a hash-routed layer needs the ids
