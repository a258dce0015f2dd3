"""Shared set-up for the GPU parity tests: device tensors, synthetic layers
built on the GPU with the seeded fill, and the oracle-side twin that
regenerates only the experts a call actually uses.

Expected values always come from ``oracle`` on inputs produced by ``synth``
(never from the HIP path)."""
from __future__ import annotations

import copy

import numpy as np
import torch

import oracle
import quantized_moe_decode_route_amd as moe
import synth

BLOCK = {"mxfp4": (32, 17), "q2k": (256, 84)}


def dev(a: np.ndarray) -> torch.Tensor:
    """numpy -> device tensor with the same bytes (uint16 travels as int16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    elif a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a.copy()).to("cuda")


def host(t: torch.Tensor, dtype=None) -> np.ndarray:
    a = t.detach().cpu().numpy()
    return a.view(dtype) if dtype is not None else a


def rel_inf_err(y_gpu: np.ndarray, y_ref: np.ndarray) -> np.ndarray:
    """Per row: max |gpu - ref| / max |ref|."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64).reshape(y_ref.shape)
    num = np.max(np.abs(y_gpu - y_ref), axis=-1)
    den = np.max(np.abs(y_ref), axis=-1)
    return num / np.where(den == 0, 1.0, den)


TOL = 1e-4  # max |err| <= 1e-4 * ||y||_inf per token, fp32-accumulated outputs


def assert_parity(y_gpu, y_ref, tol=TOL, what=""):
    e = rel_inf_err(y_gpu, y_ref)
    assert np.all(e <= tol), f"{what}: max rel-inf error {e.max():.3e} > {tol}"
    return float(e.max())


def matrix_bytes(fmt: str, n: int, k: int) -> int:
    bw, bb = BLOCK[fmt]
    return n * (k // bw) * bb


class Layer:
    """One MoE layer with E experts resident on the GPU, seeded.

    fmt "mxfp4" / "q2k": weights filled on the GPU by synth.gpu_fill.
    fmt "int4g32": MXFP4 weights filled on the GPU, then converted by
    quantize_fp4_to_int4g32 (the conversion under test elsewhere); the oracle
    side converts its own twin bytes with oracle.quantize_fp4_to_int4g32.
    ``down_fmt``: the down projection's format when it differs (per-family
    precision); ``fmt`` then covers gate and up.
    """

    def __init__(self, fmt: str, seed: int, layer: int, E: int, D: int, F: int, top_k: int = 6,
                 down_layout: str = "rows", down_fmt: str | None = None, mutate=None):
        self.fmt, self.seed, self.layer = fmt, seed, layer
        # mutate(proj, expert, bytes) -> bytes: an edit of the seeded MXFP4 or
        # Q2_K bytes applied on both sides (the device copy is then uploaded
        # from the host instead of filled on the GPU; small shapes only)
        self.mutate = mutate
        self.down_fmt = down_fmt or fmt
        self.E, self.D, self.F, self.k = E, D, F, top_k
        self.down_layout = down_layout
        self.router = synth.router_weights(seed, layer, E, D)
        self.router_dev = dev(self.router)
        self.pfmt = {synth.PROJ_GATE: fmt, synth.PROJ_UP: fmt, synth.PROJ_DOWN: self.down_fmt}
        self.shape = {synth.PROJ_GATE: (F, D), synth.PROJ_UP: (F, D), synth.PROJ_DOWN: (D, F)}
        stream = torch.cuda.current_stream().cuda_stream
        self.w = {}  # projection -> (base, stride, scale base or None, scale stride)
        for proj in (synth.PROJ_GATE, synth.PROJ_UP, synth.PROJ_DOWN):
            pf = self.pfmt[proj]
            src = "mxfp4" if pf == "int4g32" else pf
            n, kk = self.shape[proj]
            per = matrix_bytes(src, n, kk)
            stride = (per + 255) // 256 * 256
            buf = torch.empty(E * stride, dtype=torch.uint8, device="cuda")
            bw, bb = BLOCK[src]
            for e in range(E):
                if mutate is None:
                    synth.gpu_fill(src, buf.data_ptr() + e * stride, seed, layer, e, 1, proj, n * (kk // bw),
                                   stream)
                else:
                    hb = mutate(proj, e, synth.expert_tensor(src, seed, layer, e, proj, n, kk).copy())
                    buf[e * stride:e * stride + hb.size].copy_(torch.from_numpy(hb))
            tiled = proj == synth.PROJ_DOWN and down_layout != "rows"
            if pf == "int4g32":
                qstride = n * kk // 2
                sstride = (n * (kk // 32) * 2 + 255) // 256 * 256
                q = torch.empty(E * qstride, dtype=torch.uint8, device="cuda")
                sc = torch.empty(E * sstride, dtype=torch.uint8, device="cuda")
                for e in range(E):
                    moe.quantize_fp4_to_int4g32(buf.data_ptr() + e * stride, n, kk, q.data_ptr() + e * qstride,
                                                sc.data_ptr() + e * sstride)
                del buf
                if tiled:  # same buffers' shapes, blocks permuted per expert
                    qt, st = torch.empty_like(q), torch.empty_like(sc)
                    for e in range(E):
                        moe.moe_tile_weights("int4g32", q.data_ptr() + e * qstride, n, kk,
                                             qt.data_ptr() + e * qstride, src_scale=sc.data_ptr() + e * sstride,
                                             dst_scale=st.data_ptr() + e * sstride)
                    q, sc = qt, st
                self.w[proj] = (q, qstride, sc, sstride)
            else:
                if tiled:
                    bt = torch.empty_like(buf)
                    for e in range(E):
                        if down_layout == "tile256":
                            moe.moe_tile_weights(pf, buf.data_ptr() + e * stride, n, kk, bt.data_ptr() + e * stride)
                        else:
                            moe.moe_tile_weights_mfma16(buf.data_ptr() + e * stride, n, kk,
                                                        bt.data_ptr() + e * stride)
                    buf = bt
                self.w[proj] = (buf, stride, None, 0)
        torch.cuda.synchronize()
        g, u, d = (self.w[p] for p in (synth.PROJ_GATE, synth.PROJ_UP, synth.PROJ_DOWN))
        self.desc = moe.make_layer_desc(
            fmt, self.router_dev, g[0], u[0], d[0], E, D, F, top_k, g[1], u[1], d[1], g[2], u[2], d[2],
            g[3], u[3], d[3], down_layout=down_layout, down_format=self.down_fmt)
        self._cache = {}

    # -- oracle side: regenerate expert e's bytes with the host twin
    def expert_host(self, e: int):
        if e in self._cache:
            return self._cache[e]
        mats = []
        for proj in (synth.PROJ_GATE, synth.PROJ_UP, synth.PROJ_DOWN):
            pf = self.pfmt[proj]
            n, kk = self.shape[proj]
            b = synth.expert_tensor("mxfp4" if pf == "int4g32" else pf, self.seed, self.layer, e, proj, n, kk)
            if self.mutate is not None:
                b = self.mutate(proj, e, b.copy())
            if pf == "int4g32":
                b = oracle.quantize_fp4_to_int4g32(b, n, kk)
            mats.append(b)
        self._cache[e] = tuple(mats)
        return self._cache[e]

    def with_router(self, wr: np.ndarray) -> "Layer":
        """The same experts under another router matrix (fp32 [E, D]): a new
        descriptor pointing at a device copy of ``wr``, which the oracle side
        uses too.  The expert tensors and the oracle's expert cache are shared."""
        other = copy.copy(self)
        other.router = np.ascontiguousarray(wr, dtype=np.float32)
        assert other.router.shape == (self.E, self.D)
        other.router_dev = dev(other.router)
        other.desc = type(self.desc).from_buffer_copy(self.desc)
        other.desc.router_w = other.router_dev.data_ptr()
        return other

    def workspace(self, B: int) -> torch.Tensor:
        nbytes = moe.moe_layer_workspace_bytes(B, self.D, self.F, self.E, self.k)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        assert ws.data_ptr() % 256 == 0
        moe.moe_workspace_init(ws)
        return ws

    def run(self, x_bf16: np.ndarray, ws=None):
        B = x_bf16.shape[0]
        ws = ws if ws is not None else self.workspace(B)
        x = dev(x_bf16)
        y = torch.empty((B, self.D), dtype=torch.float32, device="cuda")
        idx = torch.empty((B, self.k), dtype=torch.int32, device="cuda")
        gw = torch.empty((B, self.k), dtype=torch.float32, device="cuda")
        moe.moe_layer_decode(self.desc, x, y, ws, idx, gw)
        torch.cuda.synchronize()
        # counter slot 63 of the workspace flags a bounded wait that gave up
        assert host(ws[63 * 4:64 * 4]).view(np.uint32)[0] == 0, "a wait in the layer kernel timed out"
        return host(y), host(idx), host(gw)

    def oracle(self, x_bf16: np.ndarray):
        return oracle.layer_decode((self.fmt, self.down_fmt), self.expert_host, self.router, x_bf16, self.k, self.F)
