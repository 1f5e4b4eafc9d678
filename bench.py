#!/usr/bin/env python3
"""Benchmark of the routed-expert MoE FFN layer on one MI355X (gfx950).

A step is one pass of the whole hot path over one batch of synthetic input:
one dsv4_moe_forward call through the library's C ABI (router S1-S2,
act_quant S3, permute S4, gate+up+SwiGLU S5, down S6, combine S7); for the
workloads whose routing is drawn, the router still runs on x first and the
drawn routing is then injected.  Inputs are resident in HBM before timing starts.
For single-token decode the step rotates over 64 seeded tokens and over
several byte-identical copies of the layer's weights at distinct addresses
(like consecutive layers of a model), so no weight byte can be served from
the 256 MB Infinity Cache.  Steps are captured once into a HIP graph and the
graph is replayed, so host launch overhead does not pace the GPU.

Prints ONE JSON line.  `value` is tokens/s of the whole step; `roofline`
describes the dominant kernel, the gate+up kernel (S5; the fused one-token
kernel when that opt-in path is measured): its algorithmic bytes (or flops)
per launch divided by its average duration, measured with HIP events that the
library records in that kernel's own dispatch over eager product steps run
back to back.  `cpu_baseline` times the oracle on a bounded sample on the
host cores.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
  python bench.py --summarize DIR --kind trace|fetch|write   (profile summaries)
"""
from __future__ import annotations

import argparse
import ctypes
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("MoE-layer tokens/s + achieved HBM GB/s (decode) / MFMA TFLOPS (prefill), "
          "% roofline")
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA, published (FP8 x FP4 runs at this rate)
PROFILES = os.path.join(ROOT, "profiles")
DOMINANT = {"fused": "decode_ffn_kernel", "gemv": "gemv_gate_up_kernel",
            "gemm": "gemm_kernel_gate_up"}


def is_dominant(kernel_name, path):
    """Does a profiler kernel name belong to the path's dominant kernel?"""
    if path in ("fused", "gemv"):
        return DOMINANT[path] in kernel_name
    # gemm_kernel<FMT, GU, TM>: the gate+up instances
    return "gemm_kernel<" in kernel_name and ", true," in kernel_name


# --------------------------------------------------------------------------
# algorithmic work
# --------------------------------------------------------------------------

def expert_bytes(wl):
    """Bytes of one expert's three matrices (codes + scales) and of its gate+up."""
    H, I = wl.H, wl.I
    if wl.fmt == "fp4":
        mat = I * H // 2 + I * H // 32
    else:
        mat = I * H + (I // 128) * (H // 128) * 4
    return 3 * mat, 2 * mat


def work(wl, ids, path):
    """Algorithmic bytes / flops of a step and of the dominant kernel: the
    gate+up kernel (on the VALU path it streams the routed experts only --
    the shared expert's gate+up runs in the front kernel), or the fused
    one-token kernel (the routed experts' gate+up and every touched expert's
    down)."""
    T, H, I, E, k = wl.T, wl.H, wl.I, wl.E, wl.k
    routed = len(set(ids.ravel().tolist()))
    touched = routed + 1                                  # + shared expert
    per_exp, per_exp_gu = expert_bytes(wl)
    R = T * k + T
    step_bytes = touched * per_exp + H * E * 2 + T * H * 2 + T * H * 2
    step_flops = 2 * 3 * H * I * R + 2 * T * H * E
    gu_exp, gu_rows = (touched, R) if path == "gemm" else (routed, T * k)
    gu_bytes = gu_exp * per_exp_gu + T * H + T * (H // 128) * 4
    gu_flops = 2 * 2 * H * I * gu_rows
    if path == "fused":
        gu_bytes += touched * (per_exp - per_exp_gu)
        gu_flops += 2 * H * I * R
    return dict(touched=touched, step_bytes=step_bytes, step_flops=step_flops,
                gu_bytes=gu_bytes, gu_flops=gu_flops, rows=R)


def src_hash():
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "bit_expert_ffn_moe_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


# --------------------------------------------------------------------------
# HIP runtime (graphs, events) through ctypes
# --------------------------------------------------------------------------

class Hip:
    def __init__(self):
        import torch  # noqa: F401  (first: its HIP runtime is the one every caller binds to)
        L = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch loaded
        vp, pvp = ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p)
        for name, args in [("hipStreamBeginCapture", [vp, ctypes.c_int]),
                           ("hipStreamEndCapture", [vp, pvp]),
                           ("hipGraphInstantiate", [pvp, vp, vp, vp, ctypes.c_size_t]),
                           ("hipGraphLaunch", [vp, vp]),
                           ("hipGraphExecDestroy", [vp]), ("hipGraphDestroy", [vp]),
                           ("hipEventCreate", [pvp]), ("hipEventRecord", [vp, vp]),
                           ("hipEventElapsedTime", [ctypes.POINTER(ctypes.c_float), vp, vp]),
                           ("hipEventDestroy", [vp]), ("hipStreamSynchronize", [vp])]:
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        self.L = L

    def ok(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed: hip error {rc}")

    def event(self):
        e = ctypes.c_void_p()
        self.ok(self.L.hipEventCreate(ctypes.byref(e)), "hipEventCreate")
        return e

    def capture(self, stream, fn):
        g = ctypes.c_void_p()
        self.ok(self.L.hipStreamBeginCapture(stream, 2), "hipStreamBeginCapture")  # relaxed
        try:
            fn()
        finally:
            self.ok(self.L.hipStreamEndCapture(stream, ctypes.byref(g)), "hipStreamEndCapture")
        ex = ctypes.c_void_p()
        self.ok(self.L.hipGraphInstantiate(ctypes.byref(ex), g, None, None, 0),
                "hipGraphInstantiate")
        return g, ex

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        self.ok(self.L.hipEventElapsedTime(ctypes.byref(ms), a, b), "hipEventElapsedTime")
        return ms.value


# --------------------------------------------------------------------------
# the step
# --------------------------------------------------------------------------

class Bench:
    def __init__(self, wl_name, copies, n_tokens_pool, over=None, fused=False):
        import numpy as np
        import torch

        import bit_expert_ffn_moe_amd as moe
        import synth

        self.torch, self.moe, self.np = torch, moe, np
        import dataclasses
        self.wl = dataclasses.replace(synth.WORKLOADS[wl_name], **(over or {}))
        wl = self.wl
        self.pool = wl.T == 1                    # one token per step, from a pool of seeded tokens
        L = synth.make_layer(wl, **(dict(T=n_tokens_pool) if self.pool else {}))
        self.layer = L
        dev = "cuda:0"
        self.stream = torch.cuda.Stream()
        self.sp = self.stream.cuda_stream
        with torch.cuda.stream(self.stream):
            up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
            self.x_all = up(L.x)
            self.wr = up(L.wr)
            base = {n: up(getattr(L, n)) for n in
                    ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")}
            self.copies = [base] + [{n: t.clone() for n, t in base.items()}
                                    for _ in range(copies - 1)]
            fmt = (moe.MOE_W_FP4_E2M1_UE8M0_K32 if wl.fmt == "fp4"
                   else moe.MOE_W_FP8_E4M3_F32_B128)
            self.w = [moe.make_weights(fmt, wl.E, wl.H, wl.I, c["gate_q"], c["gate_s"],
                                       c["up_q"], c["up_s"], c["down_q"], c["down_s"])
                      for c in self.copies]
            T, H, k, E = wl.T, wl.H, wl.k, wl.E
            self.T = T
            self.ws_bytes = moe.moe_workspace_bytes(self.w[0], T, k)
            self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
            moe.moe_workspace_init(self.ws, self.ws_bytes, self.sp)
            i32, f32 = torch.int32, torch.float32
            self.ids = torch.empty((T, k), dtype=i32, device=dev)
            self.tw = torch.empty((T, k), dtype=f32, device=dev)
            self.inj_ids = up(L.ids) if L.ids is not None else None
            self.inj_w = up(L.w) if L.w is not None else None
            self.xq = torch.empty((T, H), dtype=torch.uint8, device=dev)
            self.xs = torch.empty((T, H // 128), dtype=f32, device=dev)
            self.offsets = torch.empty(E + 2, dtype=i32, device=dev)
            R = T * k + T
            self.row_token = torch.empty(R, dtype=i32, device=dev)
            self.row_of = torch.empty((T, k + 1), dtype=i32, device=dev)
            self.y = torch.empty((R, H), dtype=f32, device=dev)
            self.out = torch.empty((T, H), dtype=torch.uint16, device=dev)
        torch.cuda.synchronize()
        # the expert path the library takes for this shape: only the VALU
        # GEMV path keeps an fp32 h in the workspace; of it, one token with
        # FP4 weights runs the fused kernel where it fits (the library's
        # rule, checked by the fused kernel's tests through the timing hook)
        h, _, _ = moe.moe_debug_intermediates(self.w[0], T, k, self.ws, self.ws_bytes)
        self.path = "gemv" if h is not None else "gemm"
        if (self.path == "gemv" and fused and T == 1 and wl.fmt == "fp4" and k + 1 <= 8
                and I_fits(wl) and H % 16 == 0 and H <= 4096
                and H // 16 <= torch.cuda.get_device_properties(0).multi_processor_count):
            self.path = "fused"

    def x_of(self, step):
        if self.pool:
            t = step % self.x_all.shape[0]
            return self.x_all[t:t + 1]
        return self.x_all

    def product_step(self, i):
        """Enqueue step i as the product runs it: one dsv4_moe_forward call
        (router on x, or -- for drawn routing -- the router on x followed by
        the forward with the drawn routing injected)."""
        moe, wl = self.moe, self.wl
        T, H, E, k = self.T, wl.H, wl.E, wl.k
        w = self.w[i % len(self.w)]
        x = self.x_of(i)
        if self.inj_ids is not None:
            moe.moe_route(x, self.wr, T, H, E, k, self.ids, self.tw, self.ws, self.ws_bytes,
                          self.sp)
        moe.dsv4_moe_forward(w, self.wr, x, T, k, self.inj_ids, self.inj_w, self.out,
                             moe.MOE_DT_BF16, self.ws, self.ws_bytes, self.sp)


def I_fits(wl):
    return wl.I <= 2048 and wl.I % 128 == 0


def kernel_ids(moe, path):
    """(dominant, down) kernel ids of the timing hook for the path (the fused
    kernel has no separate down)."""
    if path == "fused":
        return moe.MOE_KERNEL_DECODE_FFN, None
    if path == "gemv":
        return moe.MOE_KERNEL_GEMV_GATE_UP, moe.MOE_KERNEL_GEMV_DOWN
    return moe.MOE_KERNEL_GEMM_GATE_UP, moe.MOE_KERNEL_GEMM_DOWN


def time_kernel(B, which, n_ev):
    """Average duration (s) of kernel `which` over n_ev eager product steps,
    from HIP events the library records in that kernel's own dispatch."""
    import numpy as np
    import torch
    evs = [(B.hip.event(), B.hip.event()) for _ in range(n_ev)]
    # a bounded spin on the stream first (~20 ms), so that the steps are all
    # queued before the GPU reaches them and run back to back as in the graph
    # replays, instead of trailing the host's launches
    with torch.cuda.stream(B.stream):
        torch.cuda._sleep(50_000_000)
    for i in range(n_ev):
        B.moe.moe_debug_time_kernel(which, evs[i][0], evs[i][1])
        B.product_step(i)
    B.moe.moe_debug_time_kernel(which, None, None)
    torch.cuda.synchronize()
    ms = [B.hip.elapsed_ms(a, b) for a, b in evs]
    for a, b in evs:
        B.hip.L.hipEventDestroy(a)
        B.hip.L.hipEventDestroy(b)
    return float(np.mean(ms)) * 1e-3, float(np.percentile(ms, 10)) * 1e-3, \
        float(np.percentile(ms, 90)) * 1e-3


def measure(wl_name, steps, warmup, copies=0, graph_steps=0, hip=None, over=None, fused=False):
    """Time `steps` whole-layer steps of a workload (graph replays) and its
    dominant and down kernels; returns the figures as a dict.  `over` changes
    the workload's T or weight format (the small-batch sweep); fused=True
    runs the one-token FP4 path with the fused expert kernel (opt-in; the
    library's default is the separate gate+up and down+combine kernels)."""
    import bit_expert_ffn_moe_amd as moe
    moe.moe_debug_set_decode_fused(1 if fused else 0)
    try:
        return _measure(wl_name, steps, warmup, copies, graph_steps, hip, over, fused)
    finally:
        moe.moe_debug_set_decode_fused(0)


def _measure(wl_name, steps, warmup, copies, graph_steps, hip, over, fused):
    import dataclasses

    import numpy as np
    import torch

    import synth
    wl = dataclasses.replace(synth.WORKLOADS[wl_name], **(over or {}))
    copies = copies or (8 if wl.T == 1 else 2 if wl.T <= 64 else 1)
    B = Bench(wl_name, copies, 64, over, fused)
    B.hip = hip or Hip()
    per_graph = graph_steps or (64 if wl.T == 1 else 8 if wl.T <= 64 else 1)
    per_graph = max(1, min(per_graph, steps))
    # eager warm-up (also caches the library's one-time device check)
    for i in range(max(2, min(warmup, 16))):
        B.product_step(i)
    torch.cuda.synchronize()
    g1, ex1 = B.hip.capture(B.sp, lambda: [B.product_step(i) for i in range(per_graph)])
    reps = max(1, steps // per_graph)
    steps = reps * per_graph
    L = B.hip.L
    for _ in range(max(1, warmup // per_graph)):
        B.hip.ok(L.hipGraphLaunch(ex1, B.sp), "hipGraphLaunch")
    torch.cuda.synchronize()
    # timed region: plain graph replays, one event pair per replay as well
    ev = [B.hip.event() for _ in range(reps + 1)]
    t0 = time.perf_counter()
    B.hip.ok(L.hipEventRecord(ev[0], B.sp), "hipEventRecord")
    for r in range(reps):
        B.hip.ok(L.hipGraphLaunch(ex1, B.sp), "hipGraphLaunch")
        B.hip.ok(L.hipEventRecord(ev[r + 1], B.sp), "hipEventRecord")
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    rep_ms = [B.hip.elapsed_ms(ev[r], ev[r + 1]) / per_graph for r in range(reps)]
    for e in ev:
        L.hipEventDestroy(e)
    # with few replays in the timed region (the default 20 decode steps are one
    # graph), the spread comes from 16 more replays of the same graph after it,
    # outside the timed region
    if reps < 8:
        ev = [B.hip.event() for _ in range(17)]
        B.hip.ok(L.hipEventRecord(ev[0], B.sp), "hipEventRecord")
        for r in range(16):
            B.hip.ok(L.hipGraphLaunch(ex1, B.sp), "hipGraphLaunch")
            B.hip.ok(L.hipEventRecord(ev[r + 1], B.sp), "hipEventRecord")
        torch.cuda.synchronize()
        rep_ms += [B.hip.elapsed_ms(ev[r], ev[r + 1]) / per_graph for r in range(16)]
        for e in ev:
            L.hipEventDestroy(e)
    L.hipGraphExecDestroy(ex1)
    L.hipGraphDestroy(g1)
    n_ev = max(1, min(256 if wl.T <= 64 else 16, steps))
    gu_id, dn_id = kernel_ids(B.moe, B.path)
    gu_avg_s, gu_p10, gu_p90 = time_kernel(B, gu_id, n_ev)
    dn_avg_s = time_kernel(B, dn_id, n_ev)[0] if dn_id is not None else None
    # algorithmic work of the steps
    if wl.routing == "zipf":
        ids_steps = [B.layer.ids]
    else:
        ids_steps = []
        for i in range(min(per_graph, 64)):
            x = B.x_of(i)
            B.moe.moe_route(x, B.wr, B.T, wl.H, wl.E, wl.k, B.ids, B.tw, B.ws, B.ws_bytes, B.sp)
            torch.cuda.synchronize()
            ids_steps.append(B.ids.cpu().numpy().copy())
    works = [work(wl, ids, B.path) for ids in ids_steps]
    avg = {key: float(np.mean([w[key] for w in works])) for key in works[0]}
    ms_per_step = elapsed * 1e3 / steps
    gu_gbs = avg["gu_bytes"] / gu_avg_s / 1e9
    gu_tflops = avg["gu_flops"] / gu_avg_s / 1e12
    t_hbm = avg["gu_bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = avg["gu_flops"] / (FP8_PEAK_TFLOPS * 1e12)
    if B.path != "gemm" or t_hbm >= t_mfma:
        roof = dict(bound="hbm", achieved=round(gu_gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(gu_gbs / HBM_PEAK_GBS, 4))
    else:
        roof = dict(bound="mfma", achieved=round(gu_tflops, 2), peak=FP8_PEAK_TFLOPS,
                    unit="TFLOP/s", frac=round(gu_tflops / FP8_PEAK_TFLOPS, 4))
    kern = DOMINANT[B.path]
    roof.update(kernel=kern, kernel_avg_us=round(gu_avg_s * 1e6, 2),
                kernel_p10_us=round(gu_p10 * 1e6, 2), kernel_p90_us=round(gu_p90 * 1e6, 2),
                algorithmic_bytes=int(avg["gu_bytes"]), algorithmic_flops=int(avg["gu_flops"]),
                hbm_gbs=round(gu_gbs, 1), hbm_frac=round(gu_gbs / HBM_PEAK_GBS, 4),
                mfma_tflops=round(gu_tflops, 2),
                mfma_frac=round(gu_tflops / FP8_PEAK_TFLOPS, 4),
                traffic=traffic_from_profiles(kern, wl.name))
    step_gbs = avg["step_bytes"] / (ms_per_step * 1e-3) / 1e9
    res = dict(workload=wl.name, steps=steps, ms_per_step=round(ms_per_step, 6),
               ms_p10=round(float(np.percentile(rep_ms, 10)), 6),
               ms_p90=round(float(np.percentile(rep_ms, 90)), 6),
               tokens_per_s=round(B.T * steps / elapsed, 2), path=B.path,
               step_hbm_gbs=round(step_gbs, 1), step_roofline_frac=round(step_gbs / HBM_PEAK_GBS, 4),
               touched_experts_avg=round(avg["touched"], 2), layer_copies=copies,
               graph_steps=per_graph, roofline=roof,
               down_kernel_avg_us=None if dn_avg_s is None else round(dn_avg_s * 1e6, 2))
    if B.path == "gemm":
        # the grouped GEMM as a whole (gate+up and down): flops of every row
        ff = 2 * 3 * wl.H * wl.I * avg["rows"]
        t = gu_avg_s + dn_avg_s
        res["grouped_gemm"] = dict(gate_up_us=round(gu_avg_s * 1e6, 1),
                                   down_us=round(dn_avg_s * 1e6, 1),
                                   flops=int(ff), tflops=round(ff / t / 1e12, 1),
                                   mfma_frac=round(ff / t / 1e12 / FP8_PEAK_TFLOPS, 4))
    del B
    torch.cuda.empty_cache()
    return res


def stream_ceiling(hip, dom_bytes):
    """Plain streaming read (the library's debug read kernel) of a buffer
    the size of the dominant decode kernel's weights and of a 2 GiB buffer:
    the practical HBM read ceiling, as GB/s (best grid of a few)."""
    import torch

    import bit_expert_ffn_moe_amd as moe
    out = {}
    sink = torch.zeros(4, dtype=torch.uint8, device="cuda:0")
    L = hip.L
    for label, nbytes in ((f"{dom_bytes / 1e6:.0f}MB", dom_bytes // 16 * 16), ("2GiB", 2 << 30)):
        n_buf = max(1, min(16, (1 << 30) // nbytes)) if nbytes < (1 << 30) else 1
        bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda:0") for _ in range(n_buf)]
        best = None
        for blocks in (512, 1024, 2048, 4096):
            e0, e1 = hip.event(), hip.event()
            reps = 32 if nbytes < (1 << 30) else 4
            for i in range(4):
                moe.moe_debug_stream_read(bufs[i % n_buf], nbytes, sink, blocks)
            torch.cuda.synchronize()
            st = torch.cuda.current_stream().cuda_stream
            L.hipEventRecord(e0, st)
            for i in range(reps):
                moe.moe_debug_stream_read(bufs[i % n_buf], nbytes, sink, blocks)
            L.hipEventRecord(e1, st)
            torch.cuda.synchronize()
            gbs = nbytes * reps / (hip.elapsed_ms(e0, e1) * 1e-3) / 1e9
            best = gbs if best is None or gbs > best else best
            L.hipEventDestroy(e0)
            L.hipEventDestroy(e1)
        out[label] = round(best, 1)
        del bufs
    torch.cuda.empty_cache()
    return out


def sweep(hip):
    """Single-token decode shapes (hidden 4096, intermediate 2048, 256
    experts top-6 + shared, router on x) at T = 1 .. 256 tokens, FP4 and FP8
    weights: whole-step time, tokens/s, which expert path ran (VALU GEMV or
    MFMA grouped GEMM) and its gate+up / down kernel times."""
    out = {}
    for fmt in ("fp4", "fp8"):
        out[fmt] = {}
        for T in (1, 2, 4, 8, 16, 32, 64, 128, 256):
            print(f"# sweep {fmt} T={T}", file=sys.stderr, flush=True)
            r = measure("decode_t1", 64 if T <= 32 else 16, 8, hip=hip,
                        over=dict(T=T, fmt=fmt))
            out[fmt][T] = dict(ms_per_step=r["ms_per_step"], tokens_per_s=r["tokens_per_s"],
                               path=r["path"], gate_up_us=r["roofline"]["kernel_avg_us"],
                               down_us=r["down_kernel_avg_us"],
                               gate_up_hbm_frac=r["roofline"]["hbm_frac"])
    return out


def host_experts(hip):
    """Routed experts in pinned host memory (decode shapes: hidden 4096,
    intermediate 2048, FP4, 256 experts top-6 + shared, router on x): 64
    single-token calls through an LRU cache of n_slots expert slots in HBM,
    after 64 calls that fill it.  Each call reads its ids back to the host
    (one synchronisation) and copies its misses over PCIe on a second stream,
    computing the resident experts meanwhile.  Per n_slots: ms per token,
    hit rate, bytes copied per token and the copy rate over the timed calls."""
    import numpy as np
    import torch

    import bit_expert_ffn_moe_amd as moe
    import synth
    names = ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")
    L = synth.make_layer("decode_t1", T=64)
    wl = L.wl
    dev = "cuda:0"
    host = {n: torch.from_numpy(np.ascontiguousarray(getattr(L, n))).pin_memory() for n in names}
    fmt = moe.MOE_W_FP4_E2M1_UE8M0_K32
    host_w = moe.make_weights(fmt, wl.E, wl.H, wl.I, *[host[n] for n in names])
    x = torch.from_numpy(L.x).to(dev)
    wr = torch.from_numpy(L.wr).to(dev)
    out = torch.empty((1, wl.H), dtype=torch.uint16, device=dev)
    cs = torch.cuda.Stream()
    ev = hip.event().value
    res = {}
    for ns in (16, 64, 256):
        slots = {n: torch.empty((ns + 1,) + tuple(host[n].shape[1:]), dtype=host[n].dtype,
                                device=dev) for n in names}
        slot_w = moe.make_weights(fmt, ns, wl.H, wl.I, *[slots[n] for n in names])
        cache = moe.ExpertCache(wl.E, ns)
        wsb = moe.moe_host_experts_workspace_bytes(host_w, 1, wl.k)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        moe.moe_workspace_init(ws, wsb)
        scb = moe.moe_host_experts_scratch_bytes(wl.E, 1, wl.k)
        scratch = torch.empty(scb, dtype=torch.uint8, pin_memory=True)
        for rep in range(2):
            c0 = (cache.c.hits, cache.c.misses, cache.c.bytes_copied)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for t in range(64):
                moe.moe_forward_host_experts(host_w, slot_w, cache, wr, x[t:t + 1], 1, wl.k, out,
                                             moe.MOE_DT_BF16, ws, wsb, scratch, scb, ev,
                                             copy_stream=cs)
            torch.cuda.synchronize()
            el = time.perf_counter() - t0
        dh, dm = cache.c.hits - c0[0], cache.c.misses - c0[1]
        db = cache.c.bytes_copied - c0[2]
        res[ns] = dict(ms_per_token=round(el * 1e3 / 64, 4), tokens_per_s=round(64 / el, 1),
                       hit_rate=round(dh / max(1, dh + dm), 4),
                       mb_copied_per_token=round(db / 64 / 1e6, 2),
                       copy_gbs=round(db / el / 1e9, 2))
        del slots, ws
    torch.cuda.empty_cache()
    return res


SUB_WORKLOADS = (("tiny_t8", 256, 32), ("verify_t32", 64, 8),
                 ("prefill_fp4_t4096", 10, 3), ("prefill_fp8_t8192", 10, 3))


def run(args):
    import synth
    wl = synth.WORKLOADS[args.workload]
    hip = Hip()
    head = measure(wl.name, args.steps, args.warmup, args.copies, args.graph_steps, hip)
    if wl.T == 1 and wl.fmt == "fp4":
        # the same steps with the fused one-token expert kernel (opt-in)
        print("# one-token path with the fused expert kernel", file=sys.stderr, flush=True)
        fu = measure(wl.name, min(args.steps, 1024), args.warmup, args.copies,
                     args.graph_steps, hip, fused=True)
        if fu["path"] == "fused":
            head["fused_kernel"] = dict(
                ms_per_step=fu["ms_per_step"], tokens_per_s=fu["tokens_per_s"],
                kernel_avg_us=fu["roofline"]["kernel_avg_us"],
                algorithmic_bytes=fu["roofline"]["algorithmic_bytes"],
                hbm_gbs=fu["roofline"]["hbm_gbs"], hbm_frac=fu["roofline"]["hbm_frac"])
    line = {
        "metric": METRIC, "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": head["steps"], "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ("fp8e4m3 x fp4e2m1, fp32 accumulate" if wl.fmt == "fp4"
                  else "fp8e4m3 x fp8e4m3, fp32 accumulate"),
        "data": "synthetic (seeded; random-init weights of the layer's shapes and formats)",
        "config": {"workload": wl.name, "tokens": wl.T, "hidden": wl.H, "inter": wl.I,
                   "experts": wl.E, "top_k": wl.k, "shared_experts": 1,
                   "weights": wl.fmt, "routing": wl.routing if wl.routing == "router"
                   else f"zipf s={wl.zipf_s} (injected)", "layer_copies": head["layer_copies"],
                   "graph_steps": head["graph_steps"],
                   "touched_experts_avg": head["touched_experts_avg"],
                   "step_hbm_gbs": head["step_hbm_gbs"],
                   "step_roofline_frac": head["step_roofline_frac"],
                   "ms_p10": head["ms_p10"], "ms_p90": head["ms_p90"],
                   "path": head["path"],
                   "down_kernel_avg_us": head["down_kernel_avg_us"],
                   "fused_kernel": head.get("fused_kernel")},
        "roofline": head["roofline"],
    }
    if not args.no_sub and args.workload == "decode_t1":
        dom = head["roofline"]["algorithmic_bytes"]
        ceil = stream_ceiling(hip, dom)
        line["hbm_read_ceiling_gbs"] = ceil
        line["roofline"]["frac_of_measured_ceiling"] = round(
            head["roofline"]["hbm_gbs"] / ceil[f"{dom / 1e6:.0f}MB"], 4)
        subs = {}
        for name, st, wu in SUB_WORKLOADS:
            print(f"# sub-workload {name}", file=sys.stderr, flush=True)
            subs[name] = measure(name, st, wu, hip=hip)
        line["workloads"] = subs
        line["small_batch_sweep"] = sweep(hip)
        print("# host-resident experts", file=sys.stderr, flush=True)
        line["host_resident_experts"] = host_experts(hip)
    line["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(wl, args)
    print(json.dumps(line), flush=True)


def traffic_from_profiles(kern, wl_name):
    """HBM bytes per launch of the dominant kernel from the committed
    FETCH_SIZE / WRITE_SIZE summaries, scaled by the copy-kernel calibration;
    None when missing or taken on other kernel sources."""
    p = os.path.join(PROFILES, f"{kern}_{wl_name}_pmc.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("src_hash") != src_hash():
        return None
    try:
        return int(d["fetch_kib"] * 1024 * d["fetch_calib"] + d["write_kib"] * 1024 * d["write_calib"])
    except KeyError:
        return None


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(wl, args):
    """The oracle as it stands, on the host cores, on a bounded sample; and
    one thread on a smaller sample."""
    import synth
    from oracle import Oracle, Weights
    nproc = os.cpu_count() or 1
    threads = min(16, nproc)
    orc = Oracle()

    def timed(n_tok, thr):
        if wl.name == "decode_t1":
            L = synth.make_layer(wl.name, T=n_tok)
            tokens = None
            sample = f"{n_tok} single-token decode forwards (router on x), all layer shapes as timed"
        else:
            L = synth.make_layer(wl.name)
            tokens = list(range(0, wl.T, max(1, wl.T // n_tok)))[:n_tok]
            sample = f"{len(tokens)} of the {wl.T} tokens of the timed batch (same weights and routing)"
        W = Weights.from_layer(L)
        t0 = time.perf_counter()
        orc.forward(W, L.wr, L.x, L.wl.k, ids=L.ids, w=L.w, tokens=tokens, threads=thr)
        el = time.perf_counter() - t0
        return n_tok / el, el, sample

    v, el, sample = timed(max(8, threads * 2), threads)
    v1, el1, sample1 = timed(2, 1)
    return {"value": round(v, 4), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": sample, "seconds": round(el, 2), "nproc": nproc,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS"), "cpu_model": _cpu_model(),
            "single_thread": {"value": round(v1, 4), "unit": "tokens/s", "seconds": round(el1, 2),
                              "sample": sample1}}


# --------------------------------------------------------------------------
# rocprofv3 summaries
# --------------------------------------------------------------------------

def summarize(args):
    import csv
    d = args.summarize
    os.makedirs(PROFILES, exist_ok=True)
    if args.kind == "trace":
        files = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
        assert files, f"no kernel_stats.csv under {d}"
        rows = list(csv.DictReader(open(files[0])))
        out = os.path.join(PROFILES, f"kernels_{args.workload}_trace.md")
        with open(out, "w") as f:
            f.write(f"# rocprofv3 kernel statistics: workload {args.workload}\n\n")
            f.write(f"Command: `{args.command}`\n\nSource hash: {src_hash()}\n\n")
            f.write("| kernel | calls | avg us | min us | max us | total % |\n|---|---|---|---|---|---|\n")
            for r in rows:
                f.write("| {} | {} | {:.2f} | {:.2f} | {:.2f} | {} |\n".format(
                    r["Name"][:90], r["Calls"], float(r["AverageNs"]) / 1e3,
                    float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
                    r.get("Percentage", "")))
        print(out)
        return
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    assert files, f"no counter_collection.csv under {d}"
    rows = list(csv.DictReader(open(files[0])))
    if args.kind == "counters":
        # per kernel: the average per dispatch of every collected counter
        per = {}
        for r in rows:
            name = r["Kernel_Name"].split("(")[0][:90]
            per.setdefault(name, {}).setdefault(r["Counter_Name"], {}).setdefault(
                r.get("Dispatch_Id", ""), 0.0)
            per[name][r["Counter_Name"]][r.get("Dispatch_Id", "")] += float(r["Counter_Value"])
        names = sorted({c for v in per.values() for c in v})
        out = os.path.join(PROFILES, f"kernels_{args.workload}_counters.md")
        with open(out, "w") as f:
            f.write(f"# rocprofv3 counters per dispatch (average): workload {args.workload}\n\n")
            f.write(f"Command: `{args.command}`\n\nSource hash: {src_hash()}\n\n")
            f.write("MfmaUtil = 100 * SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE * SIMDs), the "
                    "profiler's derived metric.\n\n")
            f.write("| kernel | dispatches | " + " | ".join(names) + " |\n")
            f.write("|---|---|" + "---|" * len(names) + "\n")
            for k, cs in per.items():
                nd = max(len(v) for v in cs.values())
                vals = []
                for c in names:
                    v = cs.get(c)
                    vals.append(f"{sum(v.values()) / len(v):.4g}" if v else "")
                f.write(f"| {k} | {nd} | " + " | ".join(vals) + " |\n")
        print(out)
        return
    counter = "FETCH_SIZE" if args.kind == "fetch" else "WRITE_SIZE"
    per = {}
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        name = r["Kernel_Name"]
        per.setdefault(name, []).append(float(r["Counter_Value"]))
    path = "gemv" if args.workload == "decode_t1" else "gemm"
    kern = DOMINANT[path]
    kv = [v for n, vs in per.items() if is_dominant(n, path) for v in vs]
    # calibration: the plain float32 add of --calib-mib MiB that bench.py runs
    # last (reads and writes calib_mib MiB each)
    cv = [v for n, vs in per.items() if "FunctorOnSelf_add<float>" in n for v in vs]
    p = os.path.join(PROFILES, f"{kern}_{args.workload}_pmc.json")
    dd = json.load(open(p)) if os.path.exists(p) else {}
    key = "fetch" if args.kind == "fetch" else "write"
    calib_bytes = args.calib_mib * 1024 * 1024
    calib = calib_bytes / (cv[-1] * 1024) if cv else None
    dd.update({f"{key}_kib": sum(kv) / max(1, len(kv)), f"{key}_calib": calib,
               f"{key}_command": args.command, "src_hash": src_hash(),
               f"{key}_dispatches": len(kv)})
    json.dump(dd, open(p, "w"), indent=1)
    md = os.path.join(PROFILES, f"kernels_{args.workload}_{counter.lower()}.md")
    with open(md, "w") as f:
        f.write(f"# rocprofv3 {counter} per dispatch: workload {args.workload}\n\n")
        f.write(f"Command: `{args.command}`\n\nSource hash: {src_hash()}\n\n")
        f.write(f"Calibration: a float32 add of {args.calib_mib} MiB reads {counter} = "
                f"{cv[-1] if cv else float('nan'):.1f} KiB -> factor {calib}\n\n")
        f.write("| kernel | dispatches | avg KiB | calibrated MB |\n|---|---|---|---|\n")
        for n, vs in per.items():
            a = sum(vs) / len(vs)
            f.write(f"| {n.split('(')[0][:80]} | {len(vs)} | {a:.1f} | "
                    f"{a * 1024 * (calib or 0) / 1e6:.3f} |\n")
    print(p, dd)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2048)
    ap.add_argument("--warmup", type=int, default=128)
    ap.add_argument("--workload", default="decode_t1")
    ap.add_argument("--copies", type=int, default=0)
    ap.add_argument("--graph-steps", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--host-experts-only", action="store_true",
                    help="run only the host-resident-experts measurement")
    ap.add_argument("--sweep-only", action="store_true",
                    help="run only the small-batch sweep (T = 1 .. 256, FP4 and FP8)")
    ap.add_argument("--no-sub", action="store_true",
                    help="time only --workload (no read ceiling, no other workloads)")
    ap.add_argument("--calib-mib", type=int, default=0,
                    help="after timing, run a plain float32 add of this many MiB (counter calibration)")
    ap.add_argument("--summarize", default=None)
    ap.add_argument("--kind", default="trace")
    ap.add_argument("--command", default="")
    args = ap.parse_args()
    if args.summarize:
        return summarize(args)
    if args.sweep_only:
        import torch  # noqa: F401
        print(json.dumps({"small_batch_sweep": sweep(Hip())}), flush=True)
        return
    if args.host_experts_only:
        import torch  # noqa: F401
        print(json.dumps({"host_resident_experts": host_experts(Hip())}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported in this build "
              "(the layer is not sharded across GPUs here).", file=sys.stderr)
        sys.exit(2)
    run(args)
    if args.calib_mib:
        import torch
        n = args.calib_mib * 1024 * 1024 // 4
        a = torch.ones(n, device="cuda:0")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        torch.add(a, 1.0, out=b)
        torch.cuda.synchronize()


if __name__ == "__main__":
    main()
