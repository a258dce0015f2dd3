"""The C-ABI library loads, exports every function include/moe_decode.h
declares, and rejects bad arguments on the host before any GPU work.  No
compute call is made here (these tests run without a GPU)."""
import ctypes
import os
import re

import pytest

import quantized_moe_decode_route_amd as moe
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "moe_decode.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(moe.LIB_PATH):
        from quantized_moe_decode_route_amd import _build
        _build.build()
    return moe.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s+([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("moe_route_topk", "moe_expert_gemv_mxfp4", "moe_expert_gemv_q2k", "moe_expert_gemv_int4g32",
                     "moe_layer_decode", "quantize_fp4_to_int4g32"):
        assert required in names
    assert set(names) == set(moe.EXPORTS), set(names) ^ set(moe.EXPORTS)


def test_trace_record_size_matches_header():
    m = re.search(r"#define MOE_TRACE_FIELDS (\d+)", open(HEADER).read())
    assert m and int(m.group(1)) == moe.TRACE_FIELDS


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_abi_version_and_status_strings(L):
    assert moe.moe_abi_version() == moe.ABI_VERSION == 7
    for st in range(8):
        assert moe.moe_status_string(st)
    assert moe.moe_status_string(0) == "ok"


def test_workspace_sizes(L):
    a = moe.moe_layer_workspace_bytes(1, 4096, 2048, 256, 6)
    b = moe.moe_layer_workspace_bytes(8, 4096, 2048, 256, 6)
    assert 0 < a < b and a % 256 == 0 and b % 256 == 0
    # h [8][6][2048] and yp [8][6][4096] fp32 dominate at B=8
    assert b >= 8 * 6 * (2048 + 4096) * 4
    assert moe.moe_layer_workspace_bytes(0, 4096, 2048, 256, 6) == 0
    assert moe.moe_route_workspace_bytes(8, 4096, 256, 6) < b
    assert moe.moe_stack_workspace_bytes(8, 4096, 2048, 256, 6) > b


FAKE = 0x1000  # a host-side stand-in address: never dereferenced by validation


def test_gemv_argument_validation_on_host(L):
    assert L.moe_expert_gemv_mxfp4(None, 8, 64, FAKE, 1, FAKE, None) == 1          # null weights
    assert L.moe_expert_gemv_mxfp4(FAKE, 8, 48, FAKE, 1, FAKE, None) == 2          # K % 32
    assert L.moe_expert_gemv_mxfp4(FAKE, 8, 64, FAKE, 9, FAKE, None) == 2          # B > 8
    assert L.moe_expert_gemv_mxfp4(FAKE, 8, 64, FAKE, 0, FAKE, None) == 2          # B < 1
    assert L.moe_expert_gemv_mxfp4(FAKE, 8, 64, FAKE + 4, 1, FAKE, None) == 6      # x misaligned
    assert L.moe_expert_gemv_q2k(FAKE, 8, 128, FAKE, 1, FAKE, None) == 2           # K % 256
    assert L.moe_expert_gemv_int4g32(FAKE + 4, FAKE, 8, 64, FAKE, 1, FAKE, None) == 6  # codes misaligned
    assert L.moe_expert_gemv_int4g32(FAKE, None, 8, 64, FAKE, 1, FAKE, None) == 1  # null scales


def test_alternative_numerics_validation_on_host(L):
    assert L.moe_q8k_quantize(None, 1, 256, FAKE, FAKE, None) == 1                  # null x
    assert L.moe_q8k_quantize(FAKE, 1, 128, FAKE, FAKE, None) == 2                  # K % 256
    assert L.moe_q8k_quantize(FAKE, 0, 256, FAKE, FAKE, None) == 2                  # B < 1
    assert L.moe_q8k_quantize(FAKE + 2, 1, 256, FAKE, FAKE, None) == 6              # x misaligned
    assert L.moe_expert_gemv_mxfp4_q8(FAKE, 8, 256, None, FAKE, 1, FAKE, None) == 1  # null q
    assert L.moe_expert_gemv_mxfp4_q8(FAKE, 8, 96, FAKE, FAKE, 1, FAKE, None) == 2   # K % 256
    assert L.moe_expert_gemv_mxfp4_q8(FAKE, 8, 256, FAKE, FAKE, 9, FAKE, None) == 2  # B > 8
    assert L.moe_expert_gemv_mxfp4_q8(FAKE, 8, 256, FAKE + 8, FAKE, 1, FAKE, None) == 6  # q misaligned
    assert L.moe_mxfp4_half_lut(None, None) == 1
    assert L.moe_mxfp4_half_lut(FAKE + 1, None) == 6
    assert L.moe_expert_gemv_mxfp4_hlut(FAKE, 8, 48, FAKE, 1, FAKE, None) == 2       # K % 32
    assert L.moe_expert_gemv_mxfp4_hlut(FAKE, 8, 64, FAKE + 4, 1, FAKE, None) == 6   # x misaligned


def test_layer_and_route_validation_on_host(L):
    d = moe.make_layer_desc("mxfp4", FAKE, FAKE, FAKE, FAKE, 256, 4096, 2048, 6, 4456704, 4456704, 4456704)
    ws_ok = 1 << 30
    assert L.moe_layer_decode(ctypes.byref(d), FAKE, 9, FAKE, FAKE, ws_ok, None, None, None) == 2   # B > 8
    assert L.moe_layer_decode(ctypes.byref(d), FAKE, 1, FAKE, None, ws_ok, None, None, None) == 5  # no ws
    assert L.moe_layer_decode(ctypes.byref(d), FAKE, 1, FAKE, FAKE + 16, ws_ok, None, None, None) == 5
    assert L.moe_layer_decode(ctypes.byref(d), FAKE, 1, FAKE, FAKE, 1024, None, None, None) == 5   # too small
    d.top_k = 9
    assert L.moe_layer_decode(ctypes.byref(d), FAKE, 1, FAKE, FAKE, ws_ok, None, None, None) == 2
    d.top_k, d.d_model = 6, 4016   # not a multiple of 32
    assert L.moe_layer_decode(ctypes.byref(d), FAKE, 1, FAKE, FAKE, ws_ok, None, None, None) == 2
    d.d_model, d.format = 4096, 1   # Q2_K needs multiples of 256: 4096 and 2048 are fine
    d.gate_stride = 2752514         # but strides must keep 4-byte alignment
    assert L.moe_layer_decode(ctypes.byref(d), FAKE, 1, FAKE, FAKE, ws_ok, None, None, None) == 6
    d.format, d.gate_stride = 2, 4194304
    assert L.moe_layer_decode(ctypes.byref(d), FAKE, 1, FAKE, FAKE, ws_ok, None, None, None) == 1  # no scales
    assert L.moe_layer_decode(None, FAKE, 1, FAKE, FAKE, ws_ok, None, None, None) == 1
    assert L.moe_route_topk(FAKE, 300, 64, FAKE, 1, 6, FAKE, FAKE, None, FAKE, ws_ok, None) == 2   # E > 256
    assert L.moe_route_topk(FAKE, 256, 64, FAKE, 1, 0, FAKE, FAKE, None, FAKE, ws_ok, None) == 2   # top_k < 1
    assert L.moe_route_topk(FAKE, 4, 64, FAKE, 1, 6, FAKE, FAKE, None, FAKE, ws_ok, None) == 2     # top_k > E
    assert L.moe_stack_decode(None, 1, FAKE, 1, FAKE, 1e-6, FAKE, ws_ok, None) == 1
    assert L.quantize_fp4_to_int4g32(FAKE, 8, 48, FAKE, FAKE, None) == 2
    assert L.quantize_fp4_to_int4g32(FAKE, 8, 64, FAKE + 4, FAKE, None) == 6
    assert L.moe_validate_mxfp4(FAKE, -1, FAKE, None) == 1
    S = L.moe_stream_read
    assert S(None, 64, 0, FAKE, None) == 1 and S(FAKE, 0, 0, FAKE, None) == 1
    assert S(FAKE, 64, 2, FAKE, None) == 1                 # not a pattern
    assert S(FAKE + 4, 64, 0, FAKE, None) == 6 and S(FAKE, 40, 0, FAKE, None) == 6
    assert S(FAKE + 2, 64, 1, FAKE, None) == 6 and S(FAKE, 16, 1, FAKE, None) == 2
    assert moe.moe_stream_mxfp4_blocks(19) == 0 and moe.moe_stream_mxfp4_blocks(20) == 1
    assert moe.moe_stream_mxfp4_blocks(17 * 128) == 128     # one 4096-column MXFP4 row


def test_mixed_format_validation_on_host(L):
    """Per-family precision: gate/up in one format, down in another."""
    d = moe.make_layer_desc("mxfp4", FAKE, FAKE, FAKE, FAKE, 256, 4096, 2048, 6, 4456704, 4456704, 2752512,
                            down_format="q2k")
    assert d.down_format == 2
    assert moe.make_layer_desc("q2k", FAKE, FAKE, FAKE, FAKE, 8, 256, 256, 2, 256, 256, 256,
                               down_format="q2k").down_format == 0        # same format: the zero default
    ws_ok = 1 << 30
    run = lambda: L.moe_layer_decode(ctypes.byref(d), FAKE, 1, FAKE, FAKE, ws_ok, None, None, None)
    d.down_format = 4                                   # not a format
    assert run() == 1
    d.down_format, d.d_ff = 2, 2080                     # Q2_K down: d_ff % 256 (and MXFP4's 32 holds)
    assert run() == 2
    d.d_ff, d.down_layout = 2048, 2                     # the matrix-core layout needs an MXFP4 down
    assert run() == 1
    d.down_layout, d.down_stride = 0, 2752514           # the down format's alignment rules
    assert run() == 6
    d.down_stride, d.down_format = 2752512, 3           # INT4 down needs its scales
    assert run() == 1


def test_hash_routing_validation_on_host(L):
    """A hash-routed layer (tid2eid set) needs the tokens' ids."""
    d = moe.make_layer_desc("mxfp4", FAKE, FAKE, FAKE, FAKE, 256, 4096, 2048, 6, 4456704, 4456704, 4456704,
                            tid2eid=FAKE, vocab=1000)
    ws_ok = 1 << 30
    layer = lambda ids: L.moe_layer_decode_ids(ctypes.byref(d), ids, FAKE, 1, FAKE, FAKE, ws_ok, None, None, None)
    assert L.moe_layer_decode(ctypes.byref(d), FAKE, 1, FAKE, FAKE, ws_ok, None, None, None) == 1  # no ids
    assert layer(None) == 1
    assert layer(FAKE + 2) == 6                                  # ids 4-byte aligned
    d.vocab = 0
    assert layer(FAKE) == 1                                      # an empty table
    d.vocab, d.tid2eid = 1000, FAKE + 2
    assert layer(FAKE) == 6                                      # table 4-byte aligned
    d.tid2eid = FAKE
    arr = (moe.moe_layer_desc * 1)(d)
    assert L.moe_stack_decode(arr, 1, FAKE, 1, FAKE, 1e-6, FAKE, ws_ok, None) == 1
    assert L.moe_stack_decode_ids(arr, 1, None, FAKE, 1, FAKE, 1e-6, FAKE, ws_ok, None) == 1
    f = ctypes.c_uint32(0)
    assert L.moe_workspace_flags(None, ws_ok, ctypes.byref(f), None) == 1
    assert L.moe_workspace_flags(FAKE + 16, ws_ok, ctypes.byref(f), None) == 5  # workspaces are 256-aligned


def test_noalloc_validation_on_host(L):
    """The static-scratch layer entry checks its arguments, and that the
    call's workspace fits the static scratch, before touching the device."""
    d = moe.make_layer_desc("mxfp4", FAKE, FAKE, FAKE, FAKE, 256, 4096, 2048, 6, 4456704, 4456704, 4456704)
    N = L.moe_layer_decode_noalloc
    assert N(None, FAKE, 1, FAKE, None, None, None) == 1
    assert N(ctypes.byref(d), None, 1, FAKE, None, None, None) == 1
    assert N(ctypes.byref(d), FAKE, 9, FAKE, None, None, None) == 2            # B > 8
    assert N(ctypes.byref(d), FAKE + 8, 1, FAKE, None, None, None) == 6        # x 16-byte aligned
    for B in range(1, 9):                                                      # the full shape fits at every B
        assert moe.moe_layer_workspace_bytes(B, 4096, 2048, 256, 6) <= moe.MOE_STATIC_SCRATCH_BYTES
    d.d_model = 8192                                                           # 12.4 MB at B = 8
    assert moe.moe_layer_workspace_bytes(8, 8192, 2048, 256, 6) > moe.MOE_STATIC_SCRATCH_BYTES
    assert N(ctypes.byref(d), FAKE, 8, FAKE, None, None, None) == moe.MOE_ERR_SCRATCH
    h = moe.make_layer_desc("mxfp4", FAKE, FAKE, FAKE, FAKE, 256, 4096, 2048, 6, 4456704, 4456704, 4456704,
                            tid2eid=FAKE, vocab=10)
    assert N(ctypes.byref(h), FAKE, 1, FAKE, None, None, None) == 1            # hash routing needs ids
    m = re.search(r"#define MOE_STATIC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == moe.MOE_STATIC_SCRATCH_BYTES


def test_layout_validation_on_host(L):
    d = moe.make_layer_desc("mxfp4", FAKE, FAKE, FAKE, FAKE, 256, 4096, 2048, 6, 4456704, 4456704, 4456704,
                            down_layout="tile256")
    ws_ok = 1 << 30
    d.down_layout = 7                                   # not a layout
    assert L.moe_layer_decode(ctypes.byref(d), FAKE, 1, FAKE, FAKE, ws_ok, None, None, None) == 1
    d.down_layout, d.d_ff = 1, 2080                     # tiles need d_ff % 256 == 0
    assert L.moe_layer_decode(ctypes.byref(d), FAKE, 1, FAKE, FAKE, ws_ok, None, None, None) == 2
    T = L.moe_tile_weights
    assert T(3, FAKE, None, 8, 256, FAKE, None, None) == 1           # bad format
    assert T(0, None, None, 8, 256, FAKE, None, None) == 1           # null source
    assert T(0, FAKE, None, 0, 256, FAKE, None, None) == 1           # N < 1
    assert T(0, FAKE, None, 8, 224, FAKE, None, None) == 2           # K % 256
    assert T(1, FAKE, None, 8, 512, FAKE + 2, None, None) == 6       # misaligned destination
    assert T(2, FAKE, None, 8, 256, FAKE, None, None) == 1           # INT4 without scales
    assert T(0, FAKE, FAKE, 8, 256, FAKE, FAKE, None) == 1           # scales only for INT4
    assert T(2, FAKE + 4, FAKE, 8, 256, FAKE, FAKE, None) == 6       # INT4 codes 16-byte aligned
    d.d_ff = 2048
    d.down_layout = 2                                   # MFMA16: MXFP4 only
    d.format = 1
    assert L.moe_layer_decode(ctypes.byref(d), FAKE, 1, FAKE, FAKE, ws_ok, None, None, None) == 1
    d.format, d.d_ff = 0, 2080                          # and d_ff % 256 == 0
    assert L.moe_layer_decode(ctypes.byref(d), FAKE, 1, FAKE, FAKE, ws_ok, None, None, None) == 2
    M = L.moe_tile_weights_mfma16
    assert M(None, 16, 256, FAKE, None) == 1                          # null source
    assert M(FAKE, 16, 224, FAKE, None) == 2                          # K % 256
    assert M(FAKE, 24, 256, FAKE, None) == 2                          # N % 16


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(moe, "_LIB", None)
    monkeypatch.setattr(moe, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError):
        moe.moe_abi_version()
