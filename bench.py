#!/usr/bin/env python3
"""Benchmark of one routed-expert MoE layer decode on one MI355X.

Workload (headline): one MoE layer, 256 experts with MXFP4 gate/up
[2048 x 4096] and down [4096 x 2048], fp32 router [256 x 4096], top-6 with
softmax, one bf16 token (B=1).  The same layer at B=8 (independent tokens,
tokens grouped per expert) is measured alongside.  Weights are seeded
synthetic bytes resident in HBM; every step uses a fresh token and the steps
rotate over several layer instances so repeated reads cannot be served by the
256 MB last-level cache.

Reported value: effective weight GB/s = algorithmic bytes per step (the
active experts' three projections read once, plus the router) / step time.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

E, D, F, TOPK = 256, 4096, 2048, 6
MX_MAT = F * (D // 32) * 17          # 4,456,448 bytes per projection
ROUTER = E * D * 4                   # 4,194,304 bytes
HBM_PEAK_GBS = 8000.0
METRIC = "effective weight GB/s (% of HBM peak) + tokens/s, MoE layer decode B=1 and B=8"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


COUNTERS_MD = os.path.join(ROOT, "profiles", "fused_layer_mxfp4_hbm_counters.md")


def kernel_source_sha256() -> str:
    import glob
    import hashlib
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "quantized_moe_decode_route_amd", "csrc", "*"))):
        h.update(os.path.basename(p).encode())
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per B=1 launch from the committed counter summary (rocprofv3
    FETCH_SIZE + WRITE_SIZE, copy-calibrated), or None when the kernel sources
    changed after the counters were taken."""
    try:
        text = open(COUNTERS_MD).read()
    except OSError:
        return None
    vals = dict(line.strip().split(": ", 1) for line in text.splitlines()
                if line.strip().startswith(("traffic_b1_bytes:", "source_sha256:")))
    if vals.get("source_sha256") != kernel_source_sha256():
        return None
    return int(vals["traffic_b1_bytes"])


def build_layers(n_layers: int, seed: int, down_layout: str = "mfma16"):
    """MXFP4 layers filled on the GPU from the seeded generator.  With
    down_layout "tile256" or "mfma16" each expert's down projection is
    permuted once into that layout (moe_tile_weights / _mfma16), as a loader
    would."""
    import torch

    import quantized_moe_decode_route_amd as moe
    import synth
    stream = torch.cuda.current_stream().cuda_stream
    layers = []
    tmp = torch.empty(E * MX_MAT, dtype=torch.uint8, device="cuda") if down_layout != "rows" else None
    for l in range(n_layers):
        mats = []
        for proj in (synth.PROJ_GATE, synth.PROJ_UP, synth.PROJ_DOWN):
            buf = torch.empty(E * MX_MAT, dtype=torch.uint8, device="cuda")
            if proj == synth.PROJ_DOWN and tmp is not None:
                synth.gpu_fill("mxfp4", tmp.data_ptr(), seed, l, 0, E, proj, F * D // 32, stream)
                for e in range(E):
                    if down_layout == "tile256":
                        moe.moe_tile_weights("mxfp4", tmp.data_ptr() + e * MX_MAT, D, F, buf.data_ptr() + e * MX_MAT)
                    else:
                        moe.moe_tile_weights_mfma16(tmp.data_ptr() + e * MX_MAT, D, F, buf.data_ptr() + e * MX_MAT)
            else:
                synth.gpu_fill("mxfp4", buf.data_ptr(), seed, l, 0, E, proj, F * D // 32, stream)
            mats.append(buf)
        router = torch.from_numpy(synth.router_weights(seed, l, E, D)).to("cuda")
        desc = moe.make_layer_desc("mxfp4", router, mats[0], mats[1], mats[2], E, D, F, TOPK,
                                   MX_MAT, MX_MAT, MX_MAT, down_layout=down_layout)
        layers.append((desc, mats, router))
    torch.cuda.synchronize()
    del tmp
    return layers


Q2K_MAT = F * (D // 256) * 84        # 2,752,512 bytes per projection (gate/up [F][D] and down [D][F])
I4_Q = F * D // 2                    # INT4 codes per projection
I4_S = F * (D // 32) * 2             # bfloat16 scales per projection
EXPERT_BYTES = {"mxfp4": 3 * MX_MAT, "q2k": 3 * Q2K_MAT, "int4g32": 3 * (I4_Q + I4_S),
                "mxfp4+q2k": 2 * MX_MAT + Q2K_MAT}


def build_format_layers(fmt: str, n_layers: int, seed: int):
    """Layers of `fmt` with 256-column tiled down projections: Q2_K filled on
    the GPU from the seeded generator; INT4 converted on the GPU from seeded
    MXFP4 experts by quantize_fp4_to_int4g32."""
    import torch

    import quantized_moe_decode_route_amd as moe
    import synth
    if fmt == "mxfp4":
        return build_layers(n_layers, seed, "mfma16")
    stream = torch.cuda.current_stream().cuda_stream
    layers = []
    if fmt == "mxfp4+q2k":  # per-family precision: MXFP4 gate/up, tiled Q2_K down
        tmp = torch.empty(E * Q2K_MAT, dtype=torch.uint8, device="cuda")
        for l in range(n_layers):
            mats = []
            for proj in (synth.PROJ_GATE, synth.PROJ_UP):
                buf = torch.empty(E * MX_MAT, dtype=torch.uint8, device="cuda")
                synth.gpu_fill("mxfp4", buf.data_ptr(), seed, l, 0, E, proj, F * D // 32, stream)
                mats.append(buf)
            buf = torch.empty(E * Q2K_MAT, dtype=torch.uint8, device="cuda")
            synth.gpu_fill("q2k", tmp.data_ptr(), seed, l, 0, E, synth.PROJ_DOWN, F * D // 256, stream)
            for e in range(E):
                moe.moe_tile_weights("q2k", tmp.data_ptr() + e * Q2K_MAT, D, F, buf.data_ptr() + e * Q2K_MAT)
            mats.append(buf)
            router = torch.from_numpy(synth.router_weights(seed, l, E, D)).to("cuda")
            desc = moe.make_layer_desc("mxfp4", router, mats[0], mats[1], mats[2], E, D, F, TOPK,
                                       MX_MAT, MX_MAT, Q2K_MAT, down_layout="tile256", down_format="q2k")
            layers.append((desc, mats, router))
    elif fmt == "q2k":
        tmp = torch.empty(E * Q2K_MAT, dtype=torch.uint8, device="cuda")
        for l in range(n_layers):
            mats = []
            for proj in (synth.PROJ_GATE, synth.PROJ_UP, synth.PROJ_DOWN):
                buf = torch.empty(E * Q2K_MAT, dtype=torch.uint8, device="cuda")
                dst = tmp if proj == synth.PROJ_DOWN else buf
                synth.gpu_fill("q2k", dst.data_ptr(), seed, l, 0, E, proj, F * D // 256, stream)
                if proj == synth.PROJ_DOWN:
                    for e in range(E):
                        moe.moe_tile_weights("q2k", tmp.data_ptr() + e * Q2K_MAT, D, F, buf.data_ptr() + e * Q2K_MAT)
                mats.append(buf)
            router = torch.from_numpy(synth.router_weights(seed, l, E, D)).to("cuda")
            desc = moe.make_layer_desc("q2k", router, mats[0], mats[1], mats[2], E, D, F, TOPK,
                                       Q2K_MAT, Q2K_MAT, Q2K_MAT, down_layout="tile256")
            layers.append((desc, mats, router))
    else:
        mx = torch.empty(E * MX_MAT, dtype=torch.uint8, device="cuda")
        tq = torch.empty(I4_Q, dtype=torch.uint8, device="cuda")
        ts = torch.empty(I4_S, dtype=torch.uint8, device="cuda")
        for l in range(n_layers):
            mats = []
            for proj, (n, kk) in ((synth.PROJ_GATE, (F, D)), (synth.PROJ_UP, (F, D)), (synth.PROJ_DOWN, (D, F))):
                synth.gpu_fill("mxfp4", mx.data_ptr(), seed, l, 0, E, proj, F * D // 32, stream)
                q = torch.empty(E * I4_Q, dtype=torch.uint8, device="cuda")
                sc = torch.empty(E * I4_S, dtype=torch.uint8, device="cuda")
                for e in range(E):
                    if proj == synth.PROJ_DOWN:
                        moe.quantize_fp4_to_int4g32(mx.data_ptr() + e * MX_MAT, n, kk, tq.data_ptr(), ts.data_ptr())
                        moe.moe_tile_weights("int4g32", tq.data_ptr(), n, kk, q.data_ptr() + e * I4_Q,
                                             src_scale=ts.data_ptr(), dst_scale=sc.data_ptr() + e * I4_S)
                    else:
                        moe.quantize_fp4_to_int4g32(mx.data_ptr() + e * MX_MAT, n, kk, q.data_ptr() + e * I4_Q,
                                                    sc.data_ptr() + e * I4_S)
                mats += [q, sc]
            router = torch.from_numpy(synth.router_weights(seed, l, E, D)).to("cuda")
            desc = moe.make_layer_desc("int4g32", router, mats[0], mats[2], mats[4], E, D, F, TOPK,
                                       I4_Q, I4_Q, I4_Q, mats[1], mats[3], mats[5], I4_S, I4_S, I4_S,
                                       down_layout="tile256")
            layers.append((desc, mats, router))
    torch.cuda.synchronize()
    return layers


def format_leg(fmt: str, n_layers: int, seed: int, steps: int, warmup: int, ws):
    """B=1 and B=8 layer throughput for one weight format (effective weight GB/s)."""
    import torch

    import quantized_moe_decode_route_amd as moe
    import synth
    log(f"{fmt}: building {n_layers} layers ...")
    layers = build_format_layers(fmt, n_layers, seed)
    out = {}
    for B in (1, 8):
        xs = [torch.from_numpy(synth.token_bf16(50000 + 97 * B + i, B, D).view(np.int16)).to("cuda")
              for i in range(warmup + steps)]
        xs_settle = [torch.from_numpy(synth.token_bf16(55000 + 97 * B + i, B, D).view(np.int16)).to("cuda")
                     for i in range(16)]
        idx_log = torch.empty((steps, B, TOPK), dtype=torch.int32, device="cuda")
        ms, _, st = time_layer(layers, xs, B, steps, warmup, ws, idx_log, xs_settle)
        U = float(np.mean([len(np.unique(r)) for r in idx_log.cpu().numpy()]))
        nbytes = U * EXPERT_BYTES[fmt] + ROUTER
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[f"b{B}"] = {"value": round(gbs, 2), "unit": "GB/s", "ms_per_step": round(ms, 5),
                        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
                        "tokens_per_s_layer": round(B * 1e3 / ms, 1), "mean_unique_experts": round(U, 2),
                        "bytes_per_step": round(nbytes), "settle": st}
    del layers
    torch.cuda.empty_cache()
    return out


def stack_leg(n_layers: int, seed: int, steps: int, warmup: int, mean_u8: float, fmt: str = "mxfp4"):
    """The residual stream through n_layers resident layers (moe_stack_decode)."""
    import torch

    import quantized_moe_decode_route_amd as moe
    import synth
    log(f"stack: building {n_layers} {fmt} layers ({n_layers * E * EXPERT_BYTES[fmt] / 1e9:.0f} GB resident) ...")
    layers = build_format_layers(fmt, n_layers, seed)
    descs = [l[0] for l in layers]
    ws = torch.empty(moe.moe_stack_workspace_bytes(8, D, F, E, TOPK), dtype=torch.uint8, device="cuda")
    moe.moe_workspace_init(ws)
    out = {"layers": n_layers, "format": fmt, "resident_bytes": n_layers * (E * EXPERT_BYTES[fmt] + ROUTER)}
    for B in (1, 8):
        hs = [torch.from_numpy(synth.token_f32(70000 + 31 * B + i, B, D)).to("cuda") for i in range(warmup + steps)]
        hs_settle = [torch.from_numpy(synth.token_f32(75000 + 31 * B + i, B, D)).to("cuda") for i in range(4)]
        hout = torch.empty((B, D), dtype=torch.float32, device="cuda")
        s = torch.cuda.current_stream().cuda_stream
        st = settle(lambda i: moe.moe_stack_decode(descs, hs_settle[i], hout, ws, stream=s), len(hs_settle))
        for i in range(warmup):
            moe.moe_stack_decode(descs, hs[i], hout, ws, stream=s)
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for i in range(steps):
            moe.moe_stack_decode(descs, hs[warmup + i], hout, ws, stream=s)
        end.record()
        torch.cuda.synchronize()
        check_flags(ws, f"stack B={B}")
        ms = start.elapsed_time(end) / steps
        u = TOPK if B == 1 else mean_u8
        nbytes = n_layers * (u * EXPERT_BYTES[fmt] + ROUTER)
        out[f"b{B}"] = {"ms_per_step": round(ms, 4), "tokens_per_s": round(B * 1e3 / ms, 1),
                        "value": round(nbytes / (ms * 1e-3) / 1e9, 2), "unit": "GB/s",
                        "bytes_per_step": round(nbytes), "settle": st,
                        "bytes_note": "exact" if B == 1 else "mean unique experts per layer taken from the B=8 layer leg"}
    del layers, descs
    torch.cuda.empty_cache()
    return out


def gemv_leg(steps: int, warmup: int, copies: int = 128):
    """Stand-alone MXFP4 matvec W [2048 x 4096] x fp32 x, rotated over `copies`
    matrices: the main path at B=1 (top-level figures), and under "numerics"
    the main path against the two alternative numerics at B=1 and B=8 -- Q8
    activations with integer dots (the quantizer launch included, and the
    matvec alone) and the binary16 table decode."""
    import torch

    import quantized_moe_decode_route_amd as moe
    import synth
    stream = torch.cuda.current_stream().cuda_stream
    w = torch.empty(copies * MX_MAT, dtype=torch.uint8, device="cuda")
    synth.gpu_fill("mxfp4", w.data_ptr(), 0x5EED + 9, 0, 0, copies, synth.PROJ_GATE, F * D // 32, stream)

    def timed(call):
        """(ms per call launched from Python, ms per call replayed from a HIP
        graph of one call per copy).  A few-microsecond kernel launched from
        Python measures the host's launch rate; the graph replay measures the
        kernels.  The replayed output is checked against the eager one."""
        for i in range(warmup):
            call(w.data_ptr() + (i % copies) * MX_MAT)
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for i in range(steps):
            call(w.data_ptr() + ((warmup + i) % copies) * MX_MAT)
        end.record()
        torch.cuda.synchronize()
        eager = start.elapsed_time(end) / steps
        call(w.data_ptr() + (copies - 1) * MX_MAT)
        torch.cuda.synchronize()
        want = call.out().clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(copies):
                call(w.data_ptr() + i * MX_MAT)
        reps = max(1, steps // copies) + 1
        g.replay()
        torch.cuda.synchronize()
        torch.cuda.synchronize()
        start.record()
        for _ in range(reps):
            g.replay()
        end.record()
        torch.cuda.synchronize()
        if not torch.equal(call.out(), want):
            log("matvec: a graph replay differs from the eager call")
            sys.exit(5)
        graph = start.elapsed_time(end) / (reps * copies)
        del g
        return eager, graph

    numerics = {}
    ms_main_b1 = None
    for B in (1, 8):
        x = torch.from_numpy(synth.token_f32(90000, B, D)).to("cuda")
        y = torch.empty((B, F), dtype=torch.float32, device="cuda")
        q = torch.empty((B, D), dtype=torch.int8, device="cuda")
        dq = torch.empty((B, D // 256), dtype=torch.float32, device="cuda")
        moe.moe_q8k_quantize(x, q, dq)

        class Call:
            def __init__(self, fn):
                self.fn = fn

            def __call__(self, wp):
                self.fn(wp)

            def out(self):
                return y

        def q8_full(wp):
            moe.moe_q8k_quantize(x, q, dq)
            moe.moe_expert_gemv_mxfp4_q8(wp, F, D, q, dq, y)

        variants = {
            "main": Call(lambda wp: moe.moe_expert_gemv_mxfp4(wp, F, D, x, y)),
            "q8_with_quantize": Call(q8_full),
            "q8_matvec_only": Call(lambda wp: moe.moe_expert_gemv_mxfp4_q8(wp, F, D, q, dq, y)),
            "half_table": Call(lambda wp: moe.moe_expert_gemv_mxfp4_hlut(wp, F, D, x, y)),
        }
        row = {}
        for name, call in variants.items():
            eager, ms = timed(call)
            if B == 1 and name == "main":
                ms_main_b1, eager_main_b1 = ms, eager
            row[name] = {"us_per_call": round(ms * 1e3, 3), "GB/s": round(MX_MAT / (ms * 1e-3) / 1e9, 2),
                         "us_per_call_python_launch": round(eager * 1e3, 3)}
        numerics[f"b{B}"] = row
    del w
    torch.cuda.empty_cache()
    gbs = MX_MAT / (ms_main_b1 * 1e-3) / 1e9
    return {"value": round(gbs, 2), "unit": "GB/s", "us_per_call": round(ms_main_b1 * 1e3, 3),
            "us_per_call_python_launch": round(eager_main_b1 * 1e3, 3),
            "timing": "HIP graph of one call per copy, replayed (kernel time incl. node dispatch)",
            "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2), "bytes_per_call": MX_MAT, "copies_rotated": copies,
            "numerics": numerics}


SETTLE_MS = 40.0          # untimed GPU work before every timed leg, whatever --warmup says
SETTLE_MIN_LAUNCHES = 64


def check_flags(ws, what: str) -> None:
    """Exit non-zero if a bounded wait in a layer kernel gave up (its results
    would be wrong) or a hash-routed layer met an invalid id."""
    import quantized_moe_decode_route_amd as moe
    f = moe.moe_workspace_flags(ws)
    if f:
        log(f"{what}: workspace flags {f:#x} (bit 0: a wait timed out; bit 1: invalid hash-routing input)")
        sys.exit(3)


def settle(launch, n_inputs: int) -> dict:
    """Runs launch(i) (i cycles over n_inputs inputs that the timed region does
    not use) until SETTLE_MS of GPU time and SETTLE_MIN_LAUNCHES launches have
    passed, so clocks and caches are in their steady state when timing starts."""
    import torch
    n, ms = 0, 0.0
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    while ms < SETTLE_MS or n < SETTLE_MIN_LAUNCHES:
        start.record()
        for _ in range(16):
            launch(n % n_inputs)
            n += 1
        end.record()
        end.synchronize()
        ms += start.elapsed_time(end)
    return {"launches": n, "ms": round(ms, 2)}


def stream_ceiling(layers, calls: int = 24):
    """Pure-read rate of the device for the layer's load patterns
    (moe_stream_read), over the resident layers' weight buffers (1.14 GB
    each, far beyond the 256 MB last-level cache): 16-byte coalesced chunks
    and 17-byte MXFP4 block windows.  GB/s counts the bytes of the range."""
    import torch

    import quantized_moe_decode_route_amd as moe
    bufs = [m for l in layers for m in l[1]]
    sink = torch.zeros(moe.MOE_STREAM_GRID, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    out = {}
    for pat in ("dwordx4", "mxfp4"):
        nbytes = bufs[0].numel() - bufs[0].numel() % 16
        for i in range(8):
            moe.moe_stream_read(bufs[i % len(bufs)], nbytes, pat, sink, stream=s)
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for i in range(calls):
            moe.moe_stream_read(bufs[(i + 3) % len(bufs)], nbytes, pat, sink, stream=s)
        end.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / calls
        out[pat] = {"GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1), "bytes_per_call": nbytes,
                    "us_per_call": round(ms * 1e3, 2)}
    return out


def int4_conversion_leg(layers):
    """quantize_fp4_to_int4g32 over one full layer: 768 MXFP4 matrices (256
    experts x gate, up, down) in three calls, one per projection."""
    import torch

    import quantized_moe_decode_route_amd as moe
    q = torch.empty(E * I4_Q, dtype=torch.uint8, device="cuda")
    sc = torch.empty(E * I4_S, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    mats = layers[0][1]
    shapes = ((E * F, D), (E * F, D), (E * D, F))   # rows of all experts, columns

    def one_layer():
        for m, (n, k) in zip(mats, shapes):
            moe.quantize_fp4_to_int4g32(m, n, k, q, sc, stream=s)
    one_layer()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 3
    start.record()
    for _ in range(reps):
        one_layer()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / reps
    bytes_in = 3 * E * MX_MAT
    bytes_out = 3 * E * (I4_Q + I4_S)
    del q, sc
    torch.cuda.empty_cache()
    return {"matrices": 3 * E, "ms_per_layer": round(ms, 3), "bytes_in": bytes_in, "bytes_out": bytes_out,
            "GB/s": round((bytes_in + bytes_out) / (ms * 1e-3) / 1e9, 1),
            "pct_hbm_peak": round(100 * (bytes_in + bytes_out) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)}


def time_layer(layers, xs, B, steps, warmup, ws, idx_log=None, xs_settle=None):
    """Average ms per step over `steps` layer launches (fresh token each, layer
    instances rotated), after a settle pass on other tokens and `warmup`
    untimed steps.  Returns (ms, host wall ms per step, settle record)."""
    import torch

    import quantized_moe_decode_route_amd as moe
    y = torch.empty((B, D), dtype=torch.float32, device="cuda")
    nl = len(layers)
    s = torch.cuda.current_stream().cuda_stream
    st = None
    if xs_settle:
        st = settle(lambda i: moe.moe_layer_decode(layers[(i + 3) % nl][0], xs_settle[i], y, ws, stream=s),
                    len(xs_settle))
    for i in range(warmup):
        moe.moe_layer_decode(layers[i % nl][0], xs[i], y, ws, stream=s)
    # The timed launches call the C entry point with prebuilt arguments (the
    # Python wrapper's per-call marshalling would otherwise rival a one-token
    # layer's GPU time); their status codes are checked after the loop.
    f = moe.lib().moe_layer_decode
    call_args = [(ctypes.byref(layers[(warmup + i) % nl][0]), xs[warmup + i].data_ptr(), B, y.data_ptr(),
                  ws.data_ptr(), ws.numel(), idx_log[i].data_ptr() if idx_log is not None else None, None, s)
                 for i in range(steps)]
    status = 0
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    start.record()
    for a in call_args:
        status |= f(*a)
    end.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    if status:
        log(f"layer B={B}: moe_layer_decode returned status {status}")
        sys.exit(4)
    check_flags(ws, f"layer B={B}")
    return start.elapsed_time(end) / steps, t_wall / steps * 1e3, st


def profile_kernel(layers, xs, B, ws):
    """Duration of each layer launch, from hipEvents recorded on the launch
    stream right before and after it (tokens of their own, not the timed
    region's)."""
    import torch

    import quantized_moe_decode_route_amd as moe
    y = torch.empty((B, D), dtype=torch.float32, device="cuda")
    nl = len(layers)
    s = torch.cuda.current_stream().cuda_stream
    n = len(xs)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
    for row in evs:
        for e in row:
            e.record()
    torch.cuda.synchronize()
    for i in range(n):
        moe.moe_layer_decode_profiled(layers[(i + 5) % nl][0], xs[i], y, ws, [e.cuda_event for e in evs[i]],
                                      stream=s)
    torch.cuda.synchronize()
    check_flags(ws, f"bracketed layer B={B}")
    return np.array([evs[i][0].elapsed_time(evs[i][1]) for i in range(n)], dtype=np.float64)


COPY_BYTES = 256 << 20


def numerics_pass(n):
    """Fixed launch order for per-kernel counters of the three matvec numerics:
    n main MXFP4 matvecs, n Q8 quantizer + integer-dot matvec pairs, n
    binary16-table matvecs, all on one W [2048 x 4096] and B=8."""
    import torch

    import quantized_moe_decode_route_amd as moe
    import synth
    stream = torch.cuda.current_stream().cuda_stream
    w = torch.empty(MX_MAT, dtype=torch.uint8, device="cuda")
    synth.gpu_fill("mxfp4", w.data_ptr(), 0x5EED + 9, 0, 0, 1, synth.PROJ_GATE, F * D // 32, stream)
    x = torch.from_numpy(synth.token_f32(90000, 8, D)).to("cuda")
    y = torch.empty((8, F), dtype=torch.float32, device="cuda")
    q = torch.empty((8, D), dtype=torch.int8, device="cuda")
    dq = torch.empty((8, D // 256), dtype=torch.float32, device="cuda")
    for _ in range(n):
        moe.moe_expert_gemv_mxfp4(w, F, D, x, y)
    for _ in range(n):
        moe.moe_q8k_quantize(x, q, dq)
        moe.moe_expert_gemv_mxfp4_q8(w, F, D, q, dq, y)
    for _ in range(n):
        moe.moe_expert_gemv_mxfp4_hlut(w, F, D, x, y)
    torch.cuda.synchronize()


def counter_pass(layers, x1, x8, ws, n, fmt="mxfp4"):
    """Fixed launch order for per-dispatch hardware counters: n B=1 layers,
    n B=8 layers, n plain device copies of COPY_BYTES (known traffic).  The
    experts the launches select are recorded, and each launch's algorithmic
    bytes (its distinct experts' three projections once, plus the router)
    are printed as one JSON line."""
    import torch

    import quantized_moe_decode_route_amd as moe
    nl = len(layers)
    alg = {}
    for B, xs in ((1, x1), (8, x8)):
        y = torch.empty((B, D), dtype=torch.float32, device="cuda")
        idx = torch.empty((n, B, TOPK), dtype=torch.int32, device="cuda")
        for i in range(n):
            moe.moe_layer_decode(layers[i % nl][0], xs[i], y, ws, idx[i])
        torch.cuda.synchronize()
        check_flags(ws, f"counter pass B={B}")
        U = [len(np.unique(r)) for r in idx.cpu().numpy()]
        alg[f"b{B}"] = {"mean_unique_experts": round(float(np.mean(U)), 3),
                        "bytes_per_launch": round(float(np.mean(U)) * EXPERT_BYTES[fmt] + ROUTER)}
    src = torch.zeros(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(n):
        torch.neg(src, out=dst)  # one elementwise kernel: reads and writes COPY_BYTES each
    torch.cuda.synchronize()
    log(f"counter pass ({fmt}): {n} x B=1 layer, {n} x B=8 layer, {n} x elementwise copy of {COPY_BYTES} bytes")
    print(json.dumps({"counter_pass": fmt, "launches": n, "copy_bytes": COPY_BYTES, **alg}), flush=True)


def cpu_baseline(seed: int, n_tokens: int):
    """The oracle on the host: B=1 layer decode of a few tokens, timed on one
    thread and on every core this process may use (threads split output rows;
    at most 16, a one-GPU host's share of its CPU)."""
    import oracle
    import synth
    wr = synth.router_weights(seed, 0, E, D)
    cache = {}

    def get(e):
        if e not in cache:
            cache[e] = tuple(synth.expert_tensor("mxfp4", seed, 0, e, p, n, k)
                             for p, (n, k) in ((0, (F, D)), (1, (F, D)), (2, (D, F))))
        return cache[e]

    xs = [synth.token_bf16(900000 + i, 1, D) for i in range(n_tokens)]
    for x in xs:  # draw the active experts' bytes before timing (input generation)
        idx, _, _ = oracle.route_topk(wr, x, TOPK)
        for e in idx[0]:
            get(int(e))
    bytes_step = TOPK * 3 * MX_MAT + ROUTER
    cores = oracle.host_cores()

    def timed(threads, toks):
        oracle.set_threads(threads)
        try:
            t = time.perf_counter()
            for x in toks:
                oracle.layer_decode("mxfp4", get, wr, x, TOPK, F)
            return (time.perf_counter() - t) / len(toks)
        finally:
            oracle.set_threads(None)

    threads = oracle.default_threads()
    dt_all = timed(threads, xs)
    dt_one = timed(1, xs[:max(1, n_tokens // 3)])
    return {"value": round(bytes_step / dt_all / 1e9, 4), "unit": "GB/s", "cores": cores, "threads": threads,
            "kind": "oracle",
            "sample": f"{n_tokens} B=1 tokens through one 256-expert MXFP4 layer (fp64 oracle on {threads} "
                      f"threads of {cores} cores, {dt_all:.3f} s per token; expert bytes drawn before timing)",
            "seconds_per_token_layer": round(dt_all, 4),
            "single_thread": {"value": round(bytes_step / dt_one / 1e9, 4), "unit": "GB/s", "threads": 1,
                              "tokens": max(1, n_tokens // 3), "seconds_per_token_layer": round(dt_one, 4)}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=8, help="layer instances the steps rotate over")
    ap.add_argument("--seed", type=int, default=0x5EED + 1)
    ap.add_argument("--cpu-tokens", type=int, default=6)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--down-layout", choices=("mfma16", "tile256", "rows"), default="mfma16",
                    help="layout of the down projections (blocks permuted once at load time)")
    ap.add_argument("--no-extra", action="store_true",
                    help="only the headline MXFP4 layer (skip the Q2_K, INT4, 43-layer stack and matvec legs)")
    ap.add_argument("--stack-layers", type=int, default=43)
    ap.add_argument("--counter-pass", type=int, default=0, metavar="N",
                    help="instead of the benchmark: N B=1 layer launches, then N B=8 launches, then N "
                         "copies of a 256 MiB buffer (the copy calibrates HBM byte counters); for "
                         "rocprofv3 --pmc runs")
    ap.add_argument("--counter-format", choices=("mxfp4", "q2k", "int4g32", "mxfp4+q2k"), default="mxfp4",
                    help="weight format of the layers in --counter-pass")
    ap.add_argument("--numerics-pass", type=int, default=0, metavar="N",
                    help="instead of the benchmark: N launches each of the main, Q8 integer-dot and "
                         "binary16-table MXFP4 matvecs (W 2048 x 4096, B=8), for rocprofv3 --pmc runs")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported (this decode path "
              f"runs on a single MI355X; there is no multi-GPU leg).", file=sys.stderr)
        sys.exit(2)

    import torch

    import quantized_moe_decode_route_amd as moe
    import synth
    torch.cuda.set_device(0)
    moe.moe_device_check()
    if args.numerics_pass:
        numerics_pass(args.numerics_pass)
        return
    if args.counter_pass and args.counter_format != "mxfp4":
        log(f"building 4 {args.counter_format} layers ...")
        layers = build_format_layers(args.counter_format, 4, args.seed + 7)
    else:
        log(f"building {args.layers} MXFP4 layers ({args.layers * 3 * E * MX_MAT / 1e9:.1f} GB) ...")
        layers = build_layers(args.layers, args.seed, args.down_layout)
    n_tok = args.warmup + args.steps
    x1 = [torch.from_numpy(synth.token_bf16(10000 + i, 1, D).view(np.int16)).to("cuda") for i in range(n_tok)]
    x8 = [torch.from_numpy(synth.token_bf16(20000 + i, 8, D).view(np.int16)).to("cuda") for i in range(n_tok)]
    ws = torch.empty(moe.moe_layer_workspace_bytes(8, D, F, E, TOPK), dtype=torch.uint8, device="cuda")
    moe.moe_workspace_init(ws)

    if args.counter_pass:
        counter_pass(layers, x1, x8, ws, args.counter_pass, args.counter_format)
        return

    x1s = [torch.from_numpy(synth.token_bf16(15000 + i, 1, D).view(np.int16)).to("cuda") for i in range(16)]
    x8s = [torch.from_numpy(synth.token_bf16(25000 + i, 8, D).view(np.int16)).to("cuda") for i in range(16)]
    log("timing B=1 ...")
    ms1, wall1, settle1 = time_layer(layers, x1, 1, args.steps, args.warmup, ws, xs_settle=x1s)
    log("timing B=8 ...")
    idx_log = torch.empty((args.steps, 8, TOPK), dtype=torch.int32, device="cuda")
    ms8, wall8, settle8 = time_layer(layers, x8, 8, args.steps, args.warmup, ws, idx_log, x8s)
    uniq = [len(np.unique(r)) for r in idx_log.cpu().numpy()]
    U8 = float(np.mean(uniq))
    bytes1 = TOPK * 3 * MX_MAT + ROUTER
    bytes8 = U8 * 3 * MX_MAT + ROUTER
    gbs1 = bytes1 / (ms1 * 1e-3) / 1e9
    gbs8 = bytes8 / (ms8 * 1e-3) / 1e9

    log("streaming-read ceiling ...")
    ceiling = stream_ceiling(layers)
    ceil_mx = ceiling["mxfp4"]["GB/s"]
    log("int4 conversion ...")
    conv = int4_conversion_leg(layers)
    log("per-kernel event timing ...")
    nb = max(args.steps, 50)
    xb1 = [torch.from_numpy(synth.token_bf16(35000 + i, 1, D).view(np.int16)).to("cuda") for i in range(nb)]
    xb8 = [torch.from_numpy(synth.token_bf16(45000 + i, 8, D).view(np.int16)).to("cuda") for i in range(nb)]
    k1s = profile_kernel(layers, xb1, 1, ws)
    k8s = profile_kernel(layers, xb8, 8, ws)
    k1, k8 = float(np.mean(k1s)), float(np.mean(k8s))

    def spread(a):
        p10, p50, p90 = np.percentile(a * 1e3, [10, 50, 90])
        return {"mean": round(float(np.mean(a)) * 1e3, 2), "p10": round(p10, 2), "p50": round(p50, 2),
                "p90": round(p90, 2)}
    # One layer launch per step: the average launch duration is the timed
    # region's HIP-event time on the launch stream divided by the launches.
    # (Events around each launch add their own marker overhead; reported as
    # launch_bracket_ms.)
    achieved = bytes1 / (ms1 * 1e-3) / 1e9

    result = {
        "metric": METRIC,
        "value": round(gbs1, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms1, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4*bf16->fp32",
        "numerics": {"weights": "mxfp4 (E2M1 codes, E8M0 scale per 32)", "x": "bf16", "router": "fp32 weights, fp64 sums",
                     "accumulate": "fp32", "h": "fp32, entering the down MFMA as six base-16 E4M3 digit terms"},
        "data": "synthetic",
        "config": {"workload": "moe_layer_decode_mxfp4_b1", "experts": E, "top_k": TOPK, "d_model": D,
                   "d_ff": F, "tokens_per_step": 1, "weight_format": "mxfp4",
                   "down_layout": args.down_layout, "layer_instances_rotated": args.layers},
        "pct_hbm_peak": round(100 * gbs1 / HBM_PEAK_GBS, 2),
        "pct_of_measured_ceiling": round(100 * gbs1 / ceil_mx, 2),
        "measured_read_ceiling": ceiling,
        "int4_conversion": conv,
        "tokens_per_s_layer": round(1e3 / ms1, 1),
        "bytes_per_step": bytes1,
        "host_wall_ms_per_step": round(wall1, 5),
        "b8": {"value": round(gbs8, 2), "unit": "GB/s", "ms_per_step": round(ms8, 5),
               "pct_hbm_peak": round(100 * gbs8 / HBM_PEAK_GBS, 2),
               "pct_of_measured_ceiling": round(100 * gbs8 / ceil_mx, 2),
               "tokens_per_s_layer": round(8e3 / ms8, 1), "mean_unique_experts": round(U8, 2),
               "bytes_per_step": round(bytes8), "host_wall_ms_per_step": round(wall8, 5), "settle": settle8},
        "settle": settle1,
        "launch_bracket_ms": {"b1": round(k1, 5), "b8": round(k8, 5)},
        "launch_bracket_us_spread": {"b1": spread(k1s), "b8": spread(k8s)},
        "roofline": {"kernel": "fused_layer_kernel (MXFP4, B=1)", "bound": "hbm", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(), "bytes_per_launch": bytes1, "launch_ms": round(ms1, 5),
                     "b8_achieved": round(gbs8, 2)},
    }
    if not args.no_extra:
        del layers
        torch.cuda.empty_cache()
        ext_steps, ext_warm = max(args.steps // 2, 10), max(args.warmup // 2, 5)
        result["formats"] = {f: format_leg(f, 4, args.seed + 7, ext_steps, ext_warm, ws)
                             for f in ("q2k", "int4g32", "mxfp4+q2k")}
        result["stack"] = stack_leg(args.stack_layers, args.seed + 11, 10, 2, U8)
        result["stack_q2k"] = stack_leg(args.stack_layers, args.seed + 13, 10, 2,
                                        result["formats"]["q2k"]["b8"]["mean_unique_experts"], fmt="q2k")
        log("matvec ...")
        result["gemv_mxfp4_2048x4096"] = gemv_leg(args.steps, args.warmup)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(args.seed, args.cpu_tokens)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
