"""CPU oracle for the routed-expert MoE decode path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package.  It shares no code with the GPU path
(``quantized_moe_decode_route_amd``) and never imports it.

The arithmetic lives in ``oracle.c`` (plain C, fp64, sequential sums); this
module loads it with ctypes and composes the per-layer and per-stack steps
with plain loops:

* ``layer_decode`` -- router logits, top-k with softmax, then for every token
  and every selected slot in rank order: gate and up matvecs, SiLU(gate)*up,
  the down matvec, and ``y[t] += g[t, j] * yp`` (fp64, slots ascending).  The
  expert FFN and its SiLU gating follow the model card
  "DeepSeek-V4-Flash-0731-W4A16" (gate/up/down projections of each routed
  expert); the router keeps the top 6 of 256 experts as "Mixed-precision
  compression of DeepSeek-V4-Flash", "The recipe", requires.
* ``stack_decode`` -- residual stream carried layer to layer with an
  unweighted RMSNorm (eps 1e-6) rounded to bfloat16 before each layer,
  starting from an fp32 residual state as the stack entry point takes it.

Every function is pinned (tests/test_oracle_pins.py); the stack by the
special cases that fix its composition (zero updates leave the residual
unchanged, the norm makes layer 0 blind to a power-of-two scale of h_0, and
equality with the explicit norm -> layer -> residual chain).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_ORACLE_LIB names another build of oracle.c (the sanitizer test's)
LIB_PATH = os.environ.get("MOE_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "oracle.c")

FMT_IDS = {"mxfp4": 0, "q2k": 1, "int4g32": 2}

_dp = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_fp = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (plain C99, no FMA contraction)."""
    if force or not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH):
        tmp = LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c99", "-D_DEFAULT_SOURCE", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-pthread", SRC_PATH, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_LIB = None


def lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        L.oracle_e2m1.restype = ctypes.c_double
        L.oracle_e2m1.argtypes = [ctypes.c_int]
        L.oracle_e8m0.restype = ctypes.c_double
        L.oracle_e8m0.argtypes = [ctypes.c_int]
        L.oracle_f16_to_double.restype = ctypes.c_double
        L.oracle_f16_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_double.restype = ctypes.c_double
        L.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_rne.restype = ctypes.c_uint16
        L.oracle_bf16_rne.argtypes = [ctypes.c_double]
        L.oracle_silu.restype = ctypes.c_double
        L.oracle_silu.argtypes = [ctypes.c_double]
        L.oracle_int4_candidate.restype = ctypes.c_float
        L.oracle_int4_candidate.argtypes = [ctypes.c_int]
        L.oracle_mxfp4_decode.restype = None
        L.oracle_mxfp4_decode.argtypes = [_u8p, ctypes.c_int64, _dp]
        L.oracle_q2k_decode.restype = None
        L.oracle_q2k_decode.argtypes = [_u8p, ctypes.c_int64, _dp]
        L.oracle_int4g32_decode.restype = None
        L.oracle_int4g32_decode.argtypes = [_i32p, _u16p, ctypes.c_int64, _dp]
        L.oracle_gemv.restype = ctypes.c_int
        L.oracle_gemv.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                  ctypes.c_int, _dp, ctypes.c_int, _dp, ctypes.c_int]
        L.oracle_dequant.restype = ctypes.c_int
        L.oracle_dequant.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                     ctypes.c_int, _dp]
        L.oracle_router_logits.restype = ctypes.c_int
        L.oracle_router_logits.argtypes = [_fp, ctypes.c_int, ctypes.c_int, _dp, ctypes.c_int, _dp,
                                           ctypes.c_int]
        L.oracle_topk_softmax.restype = ctypes.c_int
        L.oracle_topk_softmax.argtypes = [_dp, ctypes.c_int, ctypes.c_int, ctypes.c_int, _i32p, _dp]
        L.oracle_hash_route.restype = ctypes.c_int
        L.oracle_hash_route.argtypes = [_dp, ctypes.c_int, ctypes.c_int, ctypes.c_int, _i32p, ctypes.c_int, _i32p,
                                        _i32p, _dp, ctypes.POINTER(ctypes.c_int)]
        L.oracle_silu_mul.restype = None
        L.oracle_silu_mul.argtypes = [_dp, _dp, ctypes.c_int64, _dp]
        L.oracle_rmsnorm_bf16.restype = None
        L.oracle_rmsnorm_bf16.argtypes = [_dp, ctypes.c_int, ctypes.c_int, ctypes.c_double, _u16p]
        L.oracle_quantize_fp4_to_int4g32.restype = ctypes.c_int
        L.oracle_quantize_fp4_to_int4g32.argtypes = [_u8p, ctypes.c_int64, _i32p, _u16p,
                                                     ctypes.c_void_p, ctypes.c_void_p]
        _i8p = np.ctypeslib.ndpointer(dtype=np.int8, flags="C_CONTIGUOUS")
        L.oracle_q8k_quantize.restype = ctypes.c_int
        L.oracle_q8k_quantize.argtypes = [_fp, ctypes.c_int, ctypes.c_int, _i8p, _fp]
        L.oracle_gemv_mxfp4_q8.restype = ctypes.c_int
        L.oracle_gemv_mxfp4_q8.argtypes = [_u8p, ctypes.c_int, ctypes.c_int, _i8p, _fp, ctypes.c_int, _dp, _dp]
        L.oracle_mxfp4_half_lut.restype = None
        L.oracle_mxfp4_half_lut.argtypes = [_u16p]
        L.oracle_gemv_mxfp4_half.restype = ctypes.c_int
        L.oracle_gemv_mxfp4_half.argtypes = [_u8p, ctypes.c_int, ctypes.c_int, _dp, ctypes.c_int, _dp]
        _LIB = L
    return _LIB


_THREADS = None


def host_cores() -> int:
    """Cores this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count() or 1


def set_threads(n: int | None) -> None:
    """Threads the row-parallel loops use from now on (None: the default)."""
    global _THREADS
    _THREADS = None if n is None else max(1, int(n))


def default_threads() -> int:
    """The host's cores, at most 16 (a one-GPU host's share of its CPU)."""
    if _THREADS is not None:
        return _THREADS
    return max(1, min(host_cores(), 16))


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with status {rc}")


# ---------------------------------------------------------------- scalars

def e2m1(code: int) -> float:
    return lib().oracle_e2m1(int(code))


def e8m0(e: int) -> float:
    return lib().oracle_e8m0(int(e))


def f16_to_float(h: int) -> float:
    return lib().oracle_f16_to_double(int(h))


def bf16_to_float(b: int) -> float:
    return lib().oracle_bf16_to_double(int(b))


def bf16_rne(v: float) -> int:
    return int(lib().oracle_bf16_rne(float(v)))


def silu(z: float) -> float:
    return lib().oracle_silu(float(z))


def int4_candidates() -> list[float]:
    return [float(lib().oracle_int4_candidate(j)) for j in range(6)]


def bf16_array_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns to fp64 (exact), via the oracle's own decoder."""
    flat = np.asarray(bits, dtype=np.uint16).reshape(-1)
    f = lib().oracle_bf16_to_double
    return np.array([f(int(b)) for b in flat], dtype=np.float64).reshape(np.shape(bits))


def bf16_rows_to_f64(bits: np.ndarray) -> np.ndarray:
    """Fast exact widening of many bf16 values: the 16 bits become the top half
    of an IEEE binary32 pattern, which widens exactly to binary64."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- decoders

def mxfp4_decode(blocks: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(-1)
    assert b.size % 17 == 0
    n = b.size // 17
    out = np.empty(n * 32, dtype=np.float64)
    lib().oracle_mxfp4_decode(b, n, out)
    return out


def q2k_decode(blocks: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(-1)
    assert b.size % 84 == 0
    n = b.size // 84
    out = np.empty(n * 256, dtype=np.float64)
    lib().oracle_q2k_decode(b, n, out)
    return out


def int4g32_decode(q: np.ndarray, scales: np.ndarray) -> np.ndarray:
    qq = np.ascontiguousarray(q, dtype=np.int32).reshape(-1)
    ss = np.ascontiguousarray(scales, dtype=np.uint16).reshape(-1)
    assert qq.size == 4 * ss.size
    out = np.empty(ss.size * 32, dtype=np.float64)
    lib().oracle_int4g32_decode(qq, ss, ss.size, out)
    return out


# ---------------------------------------------------------------- matvec

def _weight_ptrs(fmt: str, w):
    if fmt == "int4g32":
        q, s = w
        q = np.ascontiguousarray(q, dtype=np.int32)
        s = np.ascontiguousarray(s, dtype=np.uint16)
        return (q, s), q.ctypes.data, s.ctypes.data
    b = np.ascontiguousarray(w, dtype=np.uint8)
    return (b,), b.ctypes.data, None


def gemv(fmt: str, w, n_rows: int, k: int, x: np.ndarray, nthreads: int | None = None) -> np.ndarray:
    """y[b, n] = sum_k W[n, k] x[b, k] in fp64.  ``w``: bytes (mxfp4, q2k) or (codes, scales)."""
    keep, p0, p1 = _weight_ptrs(fmt, w)
    xx = np.ascontiguousarray(np.asarray(x, dtype=np.float64).reshape(-1, k))
    B = xx.shape[0]
    y = np.empty((B, n_rows), dtype=np.float64)
    rc = lib().oracle_gemv(FMT_IDS[fmt], p0, p1, n_rows, k, xx.reshape(-1), B, y.reshape(-1),
                           nthreads or default_threads())
    _check(rc, "gemv")
    del keep
    return y


def dequant(fmt: str, w, n_rows: int, k: int) -> np.ndarray:
    keep, p0, p1 = _weight_ptrs(fmt, w)
    out = np.empty((n_rows, k), dtype=np.float64)
    _check(lib().oracle_dequant(FMT_IDS[fmt], p0, p1, n_rows, k, out.reshape(-1)), "dequant")
    del keep
    return out


# ---------------------------------------------------------------- routing

def router_logits(wr: np.ndarray, x: np.ndarray, nthreads: int | None = None) -> np.ndarray:
    wr = np.ascontiguousarray(wr, dtype=np.float32)
    E, D = wr.shape
    xx = np.ascontiguousarray(np.asarray(x, dtype=np.float64).reshape(-1, D))
    B = xx.shape[0]
    out = np.empty((B, E), dtype=np.float64)
    _check(lib().oracle_router_logits(wr.reshape(-1), E, D, xx.reshape(-1), B, out.reshape(-1),
                                      nthreads or default_threads()), "router_logits")
    return out


def topk_softmax(logits: np.ndarray, k: int) -> tuple[np.ndarray, np.ndarray]:
    l = np.ascontiguousarray(logits, dtype=np.float64)
    B, E = l.shape
    idx = np.empty((B, k), dtype=np.int32)
    g = np.empty((B, k), dtype=np.float64)
    _check(lib().oracle_topk_softmax(l.reshape(-1), E, B, k, idx.reshape(-1), g.reshape(-1)),
           "topk_softmax")
    return idx, g


def route_topk(wr: np.ndarray, x_bf16: np.ndarray, k: int = 6):
    """Returns (idx int32 [B, k], g fp64 [B, k], logits fp64 [B, E])."""
    x = bf16_rows_to_f64(x_bf16)
    logits = router_logits(wr, x)
    idx, g = topk_softmax(logits, k)
    return idx, g, logits


def hash_route(logits: np.ndarray, k: int, table: np.ndarray, ids: np.ndarray):
    """Hash-routed selection from given logits [B, E]: ``table`` int32 [vocab, k],
    ``ids`` int32 [B].  Returns (idx int32 [B, k], g fp64 [B, k], number of
    tokens with an invalid id or row, which use experts 0..k-1)."""
    l = np.ascontiguousarray(logits, dtype=np.float64)
    B, E = l.shape
    tb = np.ascontiguousarray(table, dtype=np.int32)
    iv = np.ascontiguousarray(ids, dtype=np.int32).reshape(-1)
    idx = np.empty((B, k), dtype=np.int32)
    g = np.empty((B, k), dtype=np.float64)
    nb = ctypes.c_int(0)
    _check(lib().oracle_hash_route(l.reshape(-1), E, B, k, tb.reshape(-1), tb.shape[0], iv, idx.reshape(-1),
                                   g.reshape(-1), ctypes.byref(nb)), "hash_route")
    return idx, g, nb.value


def route_hashed(wr: np.ndarray, x_bf16: np.ndarray, table: np.ndarray, ids: np.ndarray, k: int = 6):
    """Router logits as in route_topk, experts from the tid2eid table."""
    x = bf16_rows_to_f64(x_bf16)
    logits = router_logits(wr, x)
    idx, g, _ = hash_route(logits, k, table, ids)
    return idx, g, logits


def silu_mul(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    g = np.ascontiguousarray(gate, dtype=np.float64).reshape(-1)
    u = np.ascontiguousarray(up, dtype=np.float64).reshape(-1)
    h = np.empty_like(g)
    lib().oracle_silu_mul(g, u, g.size, h)
    return h.reshape(np.shape(gate))


def rmsnorm_bf16(h: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    hh = np.ascontiguousarray(h, dtype=np.float64)
    B, D = hh.shape
    out = np.empty((B, D), dtype=np.uint16)
    lib().oracle_rmsnorm_bf16(hh.reshape(-1), B, D, float(eps), out.reshape(-1))
    return out


# ---------------------------------------------------------------- expert FFN / layer

def expert_ffn(fmt, gate, up, down, x: np.ndarray, d_model: int, d_ff: int) -> np.ndarray:
    """One routed expert on one or more tokens: down(silu(gate x) * (up x)), fp64.

    ``fmt``: one format for all three projections, or (gate/up format, down
    format): precision is assigned per tensor family ("Mixed-precision
    compression of DeepSeek-V4-Flash", "The recipe")."""
    fg, fd = (fmt, fmt) if isinstance(fmt, str) else fmt
    xx = np.asarray(x, dtype=np.float64).reshape(-1, d_model)
    gv = gemv(fg, gate, d_ff, d_model, xx)
    uv = gemv(fg, up, d_ff, d_model, xx)
    h = silu_mul(gv, uv)
    return gemv(fd, down, d_model, d_ff, h)


def layer_decode(fmt, get_expert, wr: np.ndarray, x_bf16: np.ndarray, top_k: int = 6,
                 d_ff: int | None = None, hashed=None):
    """One MoE layer for B tokens (``fmt`` as in ``expert_ffn``); ``hashed``:
    (tid2eid table, token ids) for a hash-routed layer.

    ``get_expert(e)`` returns ``(gate, up, down)`` weights of expert ``e``.
    Returns ``(y fp64 [B, D], idx int32 [B, k], g fp64 [B, k])``.
    """
    E, D = wr.shape
    xb = np.asarray(x_bf16, dtype=np.uint16).reshape(-1, D)
    x = bf16_rows_to_f64(xb)
    if hashed is None:
        idx, g, _ = route_topk(wr, xb, top_k)
    else:
        idx, g, _ = route_hashed(wr, xb, hashed[0], hashed[1], top_k)
    B = x.shape[0]
    y = np.zeros((B, D), dtype=np.float64)
    cache = {}
    for t in range(B):
        for j in range(top_k):
            e = int(idx[t, j])
            if e not in cache:
                cache[e] = get_expert(e)
            gate, up, down = cache[e]
            yp = expert_ffn(fmt, gate, up, down, x[t], D, d_ff)[0]
            y[t] = y[t] + g[t, j] * yp
    return y, idx, g


def stack_decode(fmt, get_layer_expert, routers, h0: np.ndarray, top_k: int = 6,
                 d_ff: int | None = None, eps: float = 1e-6, trace: bool = False):
    """Residual stream through ``len(routers)`` layers, from the residual state
    ``h0`` ([B, D], fp32 or fp64 values, taken exactly): x_l = bf16(rmsnorm(h_l)),
    h_{l+1} = h_l + moe_l(x_l), in fp64.

    ``get_layer_expert(l, e)`` returns layer l's expert e weights.  Returns the
    final h (fp64 [B, D]) and, if ``trace``, the per-layer (x_l, idx_l, g_l, y_l).
    """
    D = routers[0].shape[1]
    h = np.array(h0, dtype=np.float64).reshape(-1, D)
    steps = []
    for l, wr in enumerate(routers):
        xl = rmsnorm_bf16(h, eps)
        y, idx, g = layer_decode(fmt, lambda e, _l=l: get_layer_expert(_l, e), wr, xl, top_k, d_ff)
        if trace:
            steps.append((xl, idx, g, y))
        h = h + y
    return (h, steps) if trace else h


# ---------------------------------------------------------------- FP4 -> INT4

def quantize_fp4_to_int4g32(mx: np.ndarray, n_rows: int, k: int, with_detail: bool = False):
    """MXFP4 [n_rows, k] bytes -> (codes int32 [n_rows, k/8], scales bf16 bits [n_rows, k/32])."""
    b = np.ascontiguousarray(mx, dtype=np.uint8).reshape(-1)
    ngroups = n_rows * (k // 32)
    assert b.size == ngroups * 17
    q = np.empty((n_rows, k // 8), dtype=np.int32)
    s = np.empty((n_rows, k // 32), dtype=np.uint16)
    s_f = np.empty(ngroups, dtype=np.float32)
    r_i = np.empty(ngroups, dtype=np.int32)
    _check(lib().oracle_quantize_fp4_to_int4g32(b, ngroups, q.reshape(-1), s.reshape(-1),
                                                s_f.ctypes.data, r_i.ctypes.data), "quantize")
    if with_detail:
        return q, s, s_f.reshape(n_rows, k // 32), r_i.reshape(n_rows, k // 32)
    return q, s


# ---------------------------------------------------------------- alternative numerics
# ("ds4.c study notes", glossary page "quantization": "MXFP4's ROCm native
# kernel" -- Q8_K activations with integer dot products; "Metal's MXFP4 ->
# half lookup table" -- exactly rounded binary16 products of scale and code.)

def q8k_quantize(x: np.ndarray):
    """fp32 activations [B, K] (K % 256 == 0) -> (q int8 [B, K], d fp32 [B, K/256]):
    per 256 activations d = fp32(max|x| / 127), q = clamp(rint(x / d), +-127) in fp32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    B, K = x.shape
    q = np.empty((B, K), dtype=np.int8)
    d = np.empty((B, K // 256), dtype=np.float32)
    _check(lib().oracle_q8k_quantize(x.reshape(-1), B, K, q.reshape(-1), d.reshape(-1)), "q8k_quantize")
    return q, d


def gemv_mxfp4_q8(blocks, n_rows: int, k: int, q: np.ndarray, d: np.ndarray):
    """MXFP4 weights [n_rows, k] against Q8 activations: (y fp64 [B, n_rows], sum of |block terms|)."""
    b = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(-1)
    q = np.ascontiguousarray(q, dtype=np.int8)
    d = np.ascontiguousarray(d, dtype=np.float32)
    B = q.shape[0]
    y = np.empty((B, n_rows), dtype=np.float64)
    a = np.empty((B, n_rows), dtype=np.float64)
    _check(lib().oracle_gemv_mxfp4_q8(b, n_rows, k, q.reshape(-1), d.reshape(-1), B, y.reshape(-1), a.reshape(-1)),
           "gemv_mxfp4_q8")
    return y, a


def mxfp4_half_lut() -> np.ndarray:
    """uint16 [256, 16]: binary16 bits of E2M1(c) * 2^(e - 127), one round-to-nearest-even."""
    out = np.empty(256 * 16, dtype=np.uint16)
    lib().oracle_mxfp4_half_lut(out)
    return out.reshape(256, 16)


def gemv_mxfp4_half(blocks, n_rows: int, k: int, x: np.ndarray) -> np.ndarray:
    """y = W x in fp64 with W decoded through ``mxfp4_half_lut``."""
    b = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(-1)
    x = np.ascontiguousarray(x, dtype=np.float64)
    B = x.shape[0]
    y = np.empty((B, n_rows), dtype=np.float64)
    _check(lib().oracle_gemv_mxfp4_half(b, n_rows, k, x.reshape(-1), B, y.reshape(-1)), "gemv_mxfp4_half")
    return y
