"""Routing edge cases through the single-launch layer at the full layer shape
(256 experts, d_model 4096, d_ff 2048, top-6), for the three weight formats
at B = 1 and B = 8, all through ``moe_layer_decode``.

The router keeps the top 6 of 256 experts ("Mixed-precision compression of
DeepSeek-V4-Flash", "The recipe"); equal logits resolve to the lower expert
index.  Three router constructions make the logits tie exactly:

* duplicated router rows: experts 128..255 come in pairs (2i, 2i+1) with
  identical rows (adjacent lanes of the top-k wave), and expert 69 repeats
  expert 5 (the same lane).  Tokens are chosen on the host so that the set
  includes an exact tie among ranks 0..3 and one across ranks 5/6 (where the
  lower index is kept and its twin dropped);
* x = 0: every logit is +-0, so experts 0..5 are selected with weight 1/6;
* six equal rows aligned with the tokens: the six largest logits are equal.

Indices must equal the oracle's bit for bit, gate weights agree within 1e-6
and outputs within 1e-4 * ||y||_inf per token."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import Layer, assert_parity

pytestmark = pytest.mark.gpu

E, D, F, K = 256, 4096, 2048, 6
FORMATS = [("mxfp4", "mfma16"), ("q2k", "tile256"), ("int4g32", "tile256")]
SIX = np.array([7, 71, 100, 131, 200, 255])  # 7 and 71 share a lane of the top-k wave

_LAYERS = {}


def layer(fmt, layout):
    key = (fmt, layout)
    if key not in _LAYERS:
        _LAYERS.clear()
        torch.cuda.empty_cache()
        _LAYERS[key] = Layer(fmt, 0x5EED + 60, 0, E, D, F, K, down_layout=layout)
    return _LAYERS[key]


def paired_router(base):
    wr = base.copy()
    wr[129:256:2] = wr[128:256:2]
    wr[69] = wr[5]
    return wr


def _sorted_logits(wr, xb):
    lg = oracle.router_logits(wr, oracle.bf16_rows_to_f64(xb))
    order = np.lexsort((np.broadcast_to(np.arange(E), lg.shape), -lg), axis=-1)
    return np.take_along_axis(lg, order, axis=-1)


def _tie_kinds(wr, xb):
    """Per token: (tie among ranks 0..3, tie across ranks 5/6)."""
    s = _sorted_logits(wr, xb)
    top = np.any(s[:, 0:3] == s[:, 1:4], axis=-1)
    boundary = s[:, 5] == s[:, 6]
    return top, boundary


def _pick_tokens(wr):
    """Deterministic token seeds: one whose top-4 holds an exact tie, one with
    an exact tie across ranks 5/6, then six more for the B = 8 batch."""
    found = {}
    for s in range(7000, 7400):
        xb = synth.token_bf16(s, 1, D)
        top, boundary = _tie_kinds(wr, xb)
        if boundary[0] and "boundary" not in found:
            found["boundary"] = xb
        elif top[0] and not boundary[0] and "top" not in found:
            found["top"] = xb
        if len(found) == 2:
            break
    assert len(found) == 2, "no token seed gives both kinds of tie"
    rest = synth.token_bf16(7500, 6, D)
    return found["top"], found["boundary"], np.concatenate([found["top"], found["boundary"], rest])


def _check(L, xb, what):
    y, idx, gw = L.run(xb)
    yo, io, go = L.oracle(xb)
    assert np.array_equal(idx, io), f"{what}: expert indices differ\n{idx}\n{io}"
    assert np.max(np.abs(gw - go)) <= 1e-6, f"{what}: gate weights differ"
    return assert_parity(y, yo, what=what), idx, gw


@pytest.mark.parametrize("fmt,layout", FORMATS)
def test_duplicated_router_rows(fmt, layout):
    L = layer(fmt, layout).with_router(paired_router(layer(fmt, layout).router))
    x_top, x_bnd, x8 = _pick_tokens(L.router)
    top, boundary = _tie_kinds(L.router, x8)
    assert top.any() and boundary.any()
    _, idx, _ = _check(L, x_top, f"{fmt} B=1 top tie")
    _, idx, _ = _check(L, x_bnd, f"{fmt} B=1 rank 5/6 tie")
    # the boundary twin with the higher index is the one left out
    s = _sorted_logits(L.router, x_bnd)[0]
    tied = np.flatnonzero(oracle.router_logits(L.router, oracle.bf16_rows_to_f64(x_bnd))[0] == s[5])
    assert tied.size >= 2 and tied[0] in idx[0] and tied[1] not in idx[0]
    err, idx8, _ = _check(L, x8, f"{fmt} B=8 duplicated rows")
    print(f"{fmt}: duplicated rows, B=8 max rel-inf err {err:.3e}, "
          f"{int(top.sum())} top ties, {int(boundary.sum())} boundary ties")


@pytest.mark.parametrize("fmt,layout", FORMATS)
def test_zero_activation(fmt, layout):
    L = layer(fmt, layout)
    x1 = np.zeros((1, D), dtype=np.uint16)
    y, idx, gw = L.run(x1)
    assert np.array_equal(idx[0], np.arange(K))
    assert np.all(np.abs(gw - 1.0 / 6.0) <= 1e-7)
    assert np.all(y == 0.0)
    # a batch mixing zero tokens with ordinary ones
    x8 = synth.token_bf16(7600, 8, D)
    x8[[0, 3, 5]] = 0
    _, idx8, gw8 = _check(L, x8, f"{fmt} B=8 with zero tokens")
    for t in (0, 3, 5):
        assert np.array_equal(idx8[t], np.arange(K))
        assert np.all(np.abs(gw8[t] - 1.0 / 6.0) <= 1e-7)


@pytest.mark.parametrize("fmt,layout", FORMATS)
@pytest.mark.parametrize("B", [1, 8])
def test_six_equal_logits(fmt, layout, B):
    base = layer(fmt, layout)
    xb = synth.token_bf16(7700 + B, B, D)
    wr = base.router.copy()
    # a row along the sum of the tokens: its logit (~41) is every token's largest
    star = (0.01 * synth.f32_from_bf16_bits(xb).astype(np.float64).sum(axis=0)).astype(np.float32)
    wr[SIX] = star
    L = base.with_router(wr)
    s = _sorted_logits(L.router, xb)
    assert np.all(s[:, :6] == s[:, :1]) and np.all(s[:, 6] < s[:, 5])
    _, idx, gw = _check(L, xb, f"{fmt} B={B} six equal logits")
    assert np.all(idx == SIX[None, :])
    assert np.all(np.abs(gw - 1.0 / 6.0) <= 1e-7)
