"""Python binding of libmoedecode.so (routed-expert MoE decode for gfx950).

Argument marshalling only: every step of the decode path runs in the HIP
kernels behind the C ABI declared in ``include/moe_decode.h``.  Functions
keep the C names; tensors are torch CUDA tensors (device memory) and the
stream defaults to torch's current stream.  If the shared library has not
been built, every call raises -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libmoedecode.so")

MOE_OK = 0
MOE_FMT_MXFP4, MOE_FMT_Q2K, MOE_FMT_INT4G32 = 0, 1, 2
FORMATS = {"mxfp4": MOE_FMT_MXFP4, "q2k": MOE_FMT_Q2K, "int4g32": MOE_FMT_INT4G32}
MOE_LAYOUT_ROWS, MOE_LAYOUT_TILE256, MOE_LAYOUT_MFMA16 = 0, 1, 2
LAYOUTS = {"rows": MOE_LAYOUT_ROWS, "tile256": MOE_LAYOUT_TILE256, "mfma16": MOE_LAYOUT_MFMA16}
# MOE_ABI_VERSION of include/moe_decode.h that this binding is written for
ABI_VERSION = 7
MOE_MAX_TOKENS = 8
MOE_MAX_TOPK = 8

EXPORTS = (
    "moe_abi_version", "moe_status_string", "moe_last_hip_error", "moe_device_check",
    "moe_expert_gemv_mxfp4", "moe_expert_gemv_q2k", "moe_expert_gemv_int4g32",
    "moe_route_workspace_bytes", "moe_route_topk",
    "moe_layer_workspace_bytes", "moe_workspace_init", "moe_layer_decode", "moe_layer_decode_ids",
    "moe_layer_decode_noalloc", "moe_workspace_flags", "moe_layer_decode_profiled", "moe_layer_decode_traced",
    "moe_stack_workspace_bytes", "moe_stack_decode", "moe_stack_decode_ids", "moe_rmsnorm_bf16",
    "quantize_fp4_to_int4g32", "moe_validate_mxfp4", "moe_tile_weights", "moe_tile_weights_mfma16",
    "moe_q8k_quantize", "moe_expert_gemv_mxfp4_q8", "moe_mxfp4_half_lut", "moe_expert_gemv_mxfp4_hlut",
    "moe_stream_read",
)


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = lib().moe_status_string(status).decode()
        if status == 4:
            msg += f" (hipError {lib().moe_last_hip_error()})"
        super().__init__(f"{fn}: status {status}: {msg}")
        self.status = status


class moe_layer_desc(ctypes.Structure):
    _fields_ = [
        ("format", ctypes.c_int), ("n_experts", ctypes.c_int), ("d_model", ctypes.c_int),
        ("d_ff", ctypes.c_int), ("top_k", ctypes.c_int),
        ("router_w", ctypes.c_void_p),
        ("gate", ctypes.c_void_p), ("up", ctypes.c_void_p), ("down", ctypes.c_void_p),
        ("gate_stride", ctypes.c_int64), ("up_stride", ctypes.c_int64), ("down_stride", ctypes.c_int64),
        ("gate_scale", ctypes.c_void_p), ("up_scale", ctypes.c_void_p), ("down_scale", ctypes.c_void_p),
        ("gate_scale_stride", ctypes.c_int64), ("up_scale_stride", ctypes.c_int64),
        ("down_scale_stride", ctypes.c_int64),
        ("down_layout", ctypes.c_int), ("down_format", ctypes.c_int),
        ("tid2eid", ctypes.c_void_p), ("vocab", ctypes.c_int),
    ]


_LIB = None
_vp, _i, _i64, _sz, _d = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_double


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(the HIP library is required; there is no fallback)")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "moe_abi_version": (_i, []),
            "moe_status_string": (ctypes.c_char_p, [_i]),
            "moe_last_hip_error": (_i, []),
            "moe_device_check": (_i, []),
            "moe_expert_gemv_mxfp4": (_i, [_vp, _i, _i, _vp, _i, _vp, _vp]),
            "moe_expert_gemv_q2k": (_i, [_vp, _i, _i, _vp, _i, _vp, _vp]),
            "moe_expert_gemv_int4g32": (_i, [_vp, _vp, _i, _i, _vp, _i, _vp, _vp]),
            "moe_q8k_quantize": (_i, [_vp, _i, _i, _vp, _vp, _vp]),
            "moe_expert_gemv_mxfp4_q8": (_i, [_vp, _i, _i, _vp, _vp, _i, _vp, _vp]),
            "moe_mxfp4_half_lut": (_i, [_vp, _vp]),
            "moe_expert_gemv_mxfp4_hlut": (_i, [_vp, _i, _i, _vp, _i, _vp, _vp]),
            "moe_route_workspace_bytes": (_sz, [_i, _i, _i, _i]),
            "moe_route_topk": (_i, [_vp, _i, _i, _vp, _i, _i, _vp, _vp, _vp, _vp, _sz, _vp]),
            "moe_layer_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
            "moe_workspace_init": (_i, [_vp, _sz, _vp]),
            "moe_layer_decode": (_i, [ctypes.POINTER(moe_layer_desc), _vp, _i, _vp, _vp, _sz, _vp, _vp, _vp]),
            "moe_layer_decode_ids": (_i, [ctypes.POINTER(moe_layer_desc), _vp, _vp, _i, _vp, _vp, _sz, _vp, _vp,
                                          _vp]),
            "moe_layer_decode_noalloc": (_i, [ctypes.POINTER(moe_layer_desc), _vp, _i, _vp, _vp, _vp, _vp]),
            "moe_workspace_flags": (_i, [_vp, _sz, ctypes.POINTER(ctypes.c_uint32), _vp]),
            "moe_layer_decode_profiled": (_i, [ctypes.POINTER(moe_layer_desc), _vp, _i, _vp, _vp, _sz, _vp, _vp,
                                               ctypes.POINTER(_vp), _vp]),
            "moe_layer_decode_traced": (_i, [ctypes.POINTER(moe_layer_desc), _vp, _i, _vp, _vp, _sz, _vp,
                                             ctypes.POINTER(_i), _vp]),
            "moe_stack_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
            "moe_stack_decode": (_i, [ctypes.POINTER(moe_layer_desc), _i, _vp, _i, _vp, _d, _vp, _sz, _vp]),
            "moe_stack_decode_ids": (_i, [ctypes.POINTER(moe_layer_desc), _i, _vp, _vp, _i, _vp, _d, _vp, _sz,
                                          _vp]),
            "moe_rmsnorm_bf16": (_i, [_vp, _i, _i, _d, _vp, _vp]),
            "quantize_fp4_to_int4g32": (_i, [_vp, _i, _i, _vp, _vp, _vp]),
            "moe_validate_mxfp4": (_i, [_vp, _i64, _vp, _vp]),
            "moe_tile_weights": (_i, [_i, _vp, _vp, _i, _i, _vp, _vp, _vp]),
            "moe_tile_weights_mfma16": (_i, [_vp, _i, _i, _vp, _vp]),
            "moe_stream_read": (_i, [_vp, _sz, _i, _vp, _vp]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _LIB = L
    return _LIB


# ---------------------------------------------------------------- marshalling helpers

def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoeError(fn, status)


# ---------------------------------------------------------------- API (C names)

def moe_abi_version() -> int:
    return lib().moe_abi_version()


def moe_status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def moe_device_check() -> None:
    _check("moe_device_check", lib().moe_device_check())


def moe_expert_gemv_mxfp4(blocks, N: int, K: int, x, y, stream=None) -> None:
    B = x.shape[0]
    _check("moe_expert_gemv_mxfp4",
           lib().moe_expert_gemv_mxfp4(_ptr(blocks), N, K, _ptr(x), B, _ptr(y), _stream(stream)))


def moe_q8k_quantize(x, q, d, stream=None) -> None:
    B, K = x.shape
    _check("moe_q8k_quantize", lib().moe_q8k_quantize(_ptr(x), B, K, _ptr(q), _ptr(d), _stream(stream)))


def moe_expert_gemv_mxfp4_q8(blocks, N: int, K: int, q, d, y, stream=None) -> None:
    B = q.shape[0]
    _check("moe_expert_gemv_mxfp4_q8",
           lib().moe_expert_gemv_mxfp4_q8(_ptr(blocks), N, K, _ptr(q), _ptr(d), B, _ptr(y), _stream(stream)))


def moe_mxfp4_half_lut(lut, stream=None) -> None:
    _check("moe_mxfp4_half_lut", lib().moe_mxfp4_half_lut(_ptr(lut), _stream(stream)))


def moe_expert_gemv_mxfp4_hlut(blocks, N: int, K: int, x, y, stream=None) -> None:
    B = x.shape[0]
    _check("moe_expert_gemv_mxfp4_hlut",
           lib().moe_expert_gemv_mxfp4_hlut(_ptr(blocks), N, K, _ptr(x), B, _ptr(y), _stream(stream)))


def moe_expert_gemv_q2k(blocks, N: int, K: int, x, y, stream=None) -> None:
    B = x.shape[0]
    _check("moe_expert_gemv_q2k",
           lib().moe_expert_gemv_q2k(_ptr(blocks), N, K, _ptr(x), B, _ptr(y), _stream(stream)))


def moe_expert_gemv_int4g32(q, scale, N: int, K: int, x, y, stream=None) -> None:
    B = x.shape[0]
    _check("moe_expert_gemv_int4g32",
           lib().moe_expert_gemv_int4g32(_ptr(q), _ptr(scale), N, K, _ptr(x), B, _ptr(y), _stream(stream)))


def moe_route_workspace_bytes(B: int, D: int, E: int, top_k: int) -> int:
    return lib().moe_route_workspace_bytes(B, D, E, top_k)


def moe_route_topk(router_w, x_bf16, top_k: int, idx, gate_w, ws, logits_out=None, stream=None) -> None:
    E, D = router_w.shape
    B = x_bf16.shape[0]
    _check("moe_route_topk",
           lib().moe_route_topk(_ptr(router_w), E, D, _ptr(x_bf16), B, top_k, _ptr(idx), _ptr(gate_w),
                                _ptr(logits_out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def moe_layer_workspace_bytes(B: int, D: int, F: int, E: int, top_k: int) -> int:
    return lib().moe_layer_workspace_bytes(B, D, F, E, top_k)


def moe_workspace_init(ws, stream=None) -> None:
    _check("moe_workspace_init",
           lib().moe_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def make_layer_desc(fmt: str, router_w, gate, up, down, n_experts: int, d_model: int, d_ff: int, top_k: int,
                    gate_stride: int, up_stride: int, down_stride: int, gate_scale=None, up_scale=None,
                    down_scale=None, gate_scale_stride: int = 0, up_scale_stride: int = 0,
                    down_scale_stride: int = 0, down_layout: str = "rows",
                    down_format: str | None = None, tid2eid=None, vocab: int = 0) -> moe_layer_desc:
    """Fill the C descriptor; tensors (or raw device addresses) must outlive its use.
    ``down_layout``: "rows" (as published), "tile256" (see moe_tile_weights) or
    "mfma16" (MXFP4 only, see moe_tile_weights_mfma16).  ``down_format``: the
    down projection's format when it differs from ``fmt`` (gate and up).  ``tid2eid``: int32
    [vocab][top_k] table of a hash-routed layer (call it through the *_ids
    entry points)."""
    d = moe_layer_desc()
    d.format = FORMATS[fmt]
    d.n_experts, d.d_model, d.d_ff, d.top_k = n_experts, d_model, d_ff, top_k
    d.router_w = _ptr(router_w)
    d.gate, d.up, d.down = _ptr(gate), _ptr(up), _ptr(down)
    d.gate_stride, d.up_stride, d.down_stride = gate_stride, up_stride, down_stride
    d.gate_scale, d.up_scale, d.down_scale = _ptr(gate_scale), _ptr(up_scale), _ptr(down_scale)
    d.gate_scale_stride, d.up_scale_stride, d.down_scale_stride = gate_scale_stride, up_scale_stride, down_scale_stride
    d.down_layout = LAYOUTS[down_layout]
    d.down_format = 0 if down_format is None or down_format == fmt else 1 + FORMATS[down_format]
    d.tid2eid, d.vocab = _ptr(tid2eid), vocab
    return d


def moe_layer_decode(desc: moe_layer_desc, x_bf16, y, ws, idx_out=None, gw_out=None, stream=None) -> None:
    B = x_bf16.shape[0]
    _check("moe_layer_decode",
           lib().moe_layer_decode(ctypes.byref(desc), _ptr(x_bf16), B, _ptr(y), _ptr(ws),
                                  ws.numel() * ws.element_size(), _ptr(idx_out), _ptr(gw_out), _stream(stream)))


def moe_layer_decode_ids(desc: moe_layer_desc, token_ids, x_bf16, y, ws, idx_out=None, gw_out=None,
                         stream=None) -> None:
    """``token_ids``: device int32 [B] (required by a hash-routed layer)."""
    B = x_bf16.shape[0]
    _check("moe_layer_decode_ids",
           lib().moe_layer_decode_ids(ctypes.byref(desc), _ptr(token_ids), _ptr(x_bf16), B, _ptr(y), _ptr(ws),
                                      ws.numel() * ws.element_size(), _ptr(idx_out), _ptr(gw_out),
                                      _stream(stream)))


MOE_ERR_SCRATCH = 7
MOE_STATIC_SCRATCH_BYTES = 8 << 20


def moe_layer_decode_noalloc(desc: moe_layer_desc, x_bf16, y, idx_out=None, gw_out=None, stream=None) -> None:
    """moe_layer_decode with the library's static per-device scratch as the
    workspace (for callers that cannot allocate)."""
    B = x_bf16.shape[0]
    _check("moe_layer_decode_noalloc",
           lib().moe_layer_decode_noalloc(ctypes.byref(desc), _ptr(x_bf16), B, _ptr(y), _ptr(idx_out), _ptr(gw_out),
                                          _stream(stream)))


def moe_workspace_flags(ws, stream=None) -> int:
    """Bit 0: a bounded wait gave up; bit 1: a hash-routed layer met an invalid id or table row."""
    f = ctypes.c_uint32(0)
    _check("moe_workspace_flags",
           lib().moe_workspace_flags(_ptr(ws), ws.numel() * ws.element_size(), ctypes.byref(f), _stream(stream)))
    return f.value


def moe_layer_decode_profiled(desc: moe_layer_desc, x_bf16, y, ws, events, idx_out=None, gw_out=None,
                              stream=None) -> None:
    """``events``: 2 raw hipEvent_t handles (ints) or None: before and after the layer."""
    B = x_bf16.shape[0]
    arr = (ctypes.c_void_p * 2)(*[e if e else None for e in events])
    _check("moe_layer_decode_profiled",
           lib().moe_layer_decode_profiled(ctypes.byref(desc), _ptr(x_bf16), B, _ptr(y), _ptr(ws),
                                           ws.numel() * ws.element_size(), _ptr(idx_out), _ptr(gw_out), arr,
                                           _stream(stream)))


TRACE_FIELDS = 16  # per workgroup: 14 time-stamp slots, XCD, XCD arrival counter


def moe_layer_decode_traced(desc: moe_layer_desc, x_bf16, y, ws, stream=None):
    """Run the layer and return per-workgroup records (int64 [blocks, 16]:
    14 slots of 100 MHz phase stamps (11 used), the XCD, the XCD arrival
    counter) as a device tensor, or None if the shape is not traced."""
    import torch
    B = x_bf16.shape[0]
    nb = ctypes.c_int(0)
    _check("moe_layer_decode_traced",
           lib().moe_layer_decode_traced(ctypes.byref(desc), _ptr(x_bf16), B, _ptr(y), _ptr(ws),
                                         ws.numel() * ws.element_size(), None, ctypes.byref(nb), _stream(stream)))
    if nb.value == 0:
        moe_layer_decode(desc, x_bf16, y, ws, stream=stream)
        return None
    tr = torch.zeros((nb.value, TRACE_FIELDS), dtype=torch.int64, device=x_bf16.device)
    _check("moe_layer_decode_traced",
           lib().moe_layer_decode_traced(ctypes.byref(desc), _ptr(x_bf16), B, _ptr(y), _ptr(ws),
                                         ws.numel() * ws.element_size(), _ptr(tr), ctypes.byref(nb),
                                         _stream(stream)))
    return tr


def moe_stack_workspace_bytes(B: int, D: int, F: int, E: int, top_k: int) -> int:
    return lib().moe_stack_workspace_bytes(B, D, F, E, top_k)


def moe_stack_decode(descs, h_in, h_out, ws, eps: float = 1e-6, stream=None) -> None:
    arr = (moe_layer_desc * len(descs))(*descs)
    B = h_in.shape[0]
    _check("moe_stack_decode",
           lib().moe_stack_decode(arr, len(descs), _ptr(h_in), B, _ptr(h_out), eps, _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream)))


def moe_stack_decode_ids(descs, token_ids, h_in, h_out, ws, eps: float = 1e-6, stream=None) -> None:
    arr = (moe_layer_desc * len(descs))(*descs)
    B = h_in.shape[0]
    _check("moe_stack_decode_ids",
           lib().moe_stack_decode_ids(arr, len(descs), _ptr(token_ids), _ptr(h_in), B, _ptr(h_out), eps, _ptr(ws),
                                      ws.numel() * ws.element_size(), _stream(stream)))


def moe_rmsnorm_bf16(h, x_out, eps: float = 1e-6, stream=None) -> None:
    B, D = h.shape
    _check("moe_rmsnorm_bf16", lib().moe_rmsnorm_bf16(_ptr(h), B, D, eps, _ptr(x_out), _stream(stream)))


def quantize_fp4_to_int4g32(mxfp4, N: int, K: int, q_out, scale_out, stream=None) -> None:
    _check("quantize_fp4_to_int4g32",
           lib().quantize_fp4_to_int4g32(_ptr(mxfp4), N, K, _ptr(q_out), _ptr(scale_out), _stream(stream)))


def moe_tile_weights(fmt: str, src, N: int, K: int, dst, src_scale=None, dst_scale=None, stream=None) -> None:
    """Row-major [N][K] weights of ``fmt`` -> the 256-column tiled layout (a block permutation)."""
    _check("moe_tile_weights",
           lib().moe_tile_weights(FORMATS[fmt], _ptr(src), _ptr(src_scale), N, K, _ptr(dst), _ptr(dst_scale),
                                  _stream(stream)))


def moe_tile_weights_mfma16(src, N: int, K: int, dst, stream=None) -> None:
    """Row-major MXFP4 [N][K] blocks -> MOE_LAYOUT_MFMA16 (a block permutation)."""
    _check("moe_tile_weights_mfma16", lib().moe_tile_weights_mfma16(_ptr(src), N, K, _ptr(dst), _stream(stream)))


def moe_validate_mxfp4(blocks, n_blocks: int, bad_count_dev, stream=None) -> None:
    _check("moe_validate_mxfp4",
           lib().moe_validate_mxfp4(_ptr(blocks), n_blocks, _ptr(bad_count_dev), _stream(stream)))


MOE_STREAM_GRID = 2048
STREAM_PATTERNS = {"dwordx4": 0, "mxfp4": 1}


def moe_stream_mxfp4_blocks(nbytes: int) -> int:
    """Blocks the MXFP4 read pattern covers in ``nbytes`` bytes (as the header's inline function)."""
    if nbytes < 20:
        return 0
    n = nbytes // 17
    while n > 0 and ((17 * (n - 1)) & ~3) + 20 > nbytes:
        n -= 1
    return n


def moe_stream_read(src, nbytes: int, pattern: str, sink, stream=None) -> None:
    """Pure-read probe: one XOR of the loaded dwords per workgroup into ``sink`` (uint32 [MOE_STREAM_GRID])."""
    _check("moe_stream_read",
           lib().moe_stream_read(_ptr(src), nbytes, STREAM_PATTERNS[pattern], _ptr(sink), _stream(stream)))
