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
describes the dominant kernel (gate+up, S5): its algorithmic bytes (or
flops) per launch divided by its average duration, measured with HIP events
on the launch stream around S5 of stage-by-stage steps that run back to back
behind a backlog of graph replays.  `cpu_baseline` times the oracle on
a bounded sample on the host cores.

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
DOMINANT = {"gemv": "gemv_gate_up_fp4_kernel", "gemm": "gemm_kernel_gate_up"}


def is_dominant(kernel_name, path):
    """Does a profiler kernel name belong to the path's dominant kernel?"""
    if path == "gemv":
        return "gemv_gate_up_fp4_kernel" in kernel_name
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
    """Algorithmic bytes / flops of a step and of the dominant kernel (the
    gate+up kernel; on the one-token VALU path it streams the routed experts
    only -- the shared expert's gate+up runs in the front kernel)."""
    T, H, I, E, k = wl.T, wl.H, wl.I, wl.E, wl.k
    routed = len(set(ids.ravel().tolist()))
    touched = routed + 1                                  # + shared expert
    per_exp, per_exp_gu = expert_bytes(wl)
    R = T * k + T
    step_bytes = touched * per_exp + H * E * 2 + T * H * 2 + T * H * 2
    step_flops = 2 * 3 * H * I * R + 2 * T * H * E
    gu_exp, gu_rows = (routed, T * k) if path == "gemv" else (touched, R)
    gu_bytes = gu_exp * per_exp_gu + T * H + T * (H // 128) * 4
    gu_flops = 2 * 2 * H * I * gu_rows
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
    def __init__(self, wl_name, copies, n_tokens_pool):
        import numpy as np
        import torch

        import bit_expert_ffn_moe_amd as moe
        import synth

        self.torch, self.moe, self.np = torch, moe, np
        over = {}
        if wl_name == "decode_t1":
            over = dict(T=n_tokens_pool)        # a pool of seeded tokens, one per step
        L = synth.make_layer(wl_name, **over)
        self.layer = L
        self.wl = synth.WORKLOADS[wl_name]
        wl = self.wl
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
        self.path = "gemv" if (wl.fmt == "fp4" and T == 1 and k + 1 <= 8) else "gemm"

    def x_of(self, step):
        if self.wl.name == "decode_t1":
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


def moe_kernel_id(moe, path):
    return moe.MOE_KERNEL_GEMV_GATE_UP if path == "gemv" else moe.MOE_KERNEL_GEMM_GATE_UP


def run(args):
    import numpy as np
    import torch

    import synth
    wl = synth.WORKLOADS[args.workload]
    copies = args.copies or (8 if wl.name == "decode_t1" else 2 if wl.T <= 64 else 1)
    B = Bench(wl.name, copies, 64)
    B.hip = Hip()
    per_graph = args.graph_steps or (64 if wl.T == 1 else 8 if wl.T <= 64 else 1)
    per_graph = max(1, min(per_graph, args.steps))
    # eager warm-up (also caches the library's one-time device check)
    for i in range(max(2, min(args.warmup, 16))):
        B.product_step(i)
    torch.cuda.synchronize()
    # graph of `per_graph` product steps
    g1, ex1 = B.hip.capture(B.sp, lambda: [B.product_step(i) for i in range(per_graph)])
    reps = max(1, args.steps // per_graph)
    steps = reps * per_graph
    wreps = max(1, args.warmup // per_graph)
    L = B.hip.L
    for _ in range(wreps):
        B.hip.ok(L.hipGraphLaunch(ex1, B.sp), "hipGraphLaunch")
    torch.cuda.synchronize()
    # timed region: plain graph replays
    t0 = time.perf_counter()
    for _ in range(reps):
        B.hip.ok(L.hipGraphLaunch(ex1, B.sp), "hipGraphLaunch")
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # dominant-kernel timing: the same product steps, run eagerly, with the
    # gate+up kernel's launches recording a pair of HIP events at that
    # kernel's own begin and end (the library's debug timing hook puts them
    # in the kernel's dispatch: no queueing gap is counted)
    n_ev = max(1, min(256, steps))
    evs = [(B.hip.event(), B.hip.event()) for _ in range(n_ev)]
    which = moe_kernel_id(B.moe, B.path)
    for i in range(n_ev):
        B.moe.moe_debug_time_kernel(which, evs[i][0], evs[i][1])
        B.product_step(i)
    B.moe.moe_debug_time_kernel(which, None, None)
    torch.cuda.synchronize()
    gu_ms = [B.hip.elapsed_ms(a, b) for a, b in evs]
    L.hipGraphExecDestroy(ex1)
    L.hipGraphDestroy(g1)
    # algorithmic work of the steps
    if wl.routing == "zipf":
        ids_steps = [B.layer.ids]
    else:
        ids_steps = []
        for i in range(per_graph):
            x = B.x_of(i)
            B.moe.moe_route(x, B.wr, B.T, wl.H, wl.E, wl.k, B.ids, B.tw, B.ws, B.ws_bytes, B.sp)
            torch.cuda.synchronize()
            ids_steps.append(B.ids.cpu().numpy().copy())
    works = [work(wl, ids, B.path) for ids in ids_steps]
    avg = {key: float(np.mean([w[key] for w in works])) for key in works[0]}
    ms_per_step = elapsed * 1e3 / steps
    value = B.T * steps / elapsed
    gu_avg_s = float(np.mean(gu_ms)) * 1e-3
    gu_gbs = avg["gu_bytes"] / gu_avg_s / 1e9
    gu_tflops = avg["gu_flops"] / gu_avg_s / 1e12
    t_hbm = avg["gu_bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = avg["gu_flops"] / (FP8_PEAK_TFLOPS * 1e12)
    if B.path == "gemv" or t_hbm >= t_mfma:
        roof = dict(bound="hbm", achieved=round(gu_gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(gu_gbs / HBM_PEAK_GBS, 4))
    else:
        roof = dict(bound="mfma", achieved=round(gu_tflops, 2), peak=FP8_PEAK_TFLOPS,
                    unit="TFLOP/s", frac=round(gu_tflops / FP8_PEAK_TFLOPS, 4))
    kern = DOMINANT[B.path]
    roof.update(kernel=kern, kernel_avg_us=round(gu_avg_s * 1e6, 2),
                algorithmic_bytes=int(avg["gu_bytes"]), algorithmic_flops=int(avg["gu_flops"]),
                mfma_tflops=round(gu_tflops, 2),
                mfma_frac=round(gu_tflops / FP8_PEAK_TFLOPS, 4),
                traffic=traffic_from_profiles(kern, wl.name))
    step_gbs = avg["step_bytes"] / (ms_per_step * 1e-3) / 1e9
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ("fp8e4m3 x fp4e2m1, fp32 accumulate" if wl.fmt == "fp4"
                  else "fp8e4m3 x fp8e4m3, fp32 accumulate"),
        "data": "synthetic (seeded; random-init weights of the layer's shapes and formats)",
        "config": {"workload": wl.name, "tokens": wl.T, "hidden": wl.H, "inter": wl.I,
                   "experts": wl.E, "top_k": wl.k, "shared_experts": 1,
                   "weights": wl.fmt, "routing": wl.routing if wl.routing == "router"
                   else f"zipf s={wl.zipf_s} (injected)", "layer_copies": copies,
                   "graph_steps": per_graph, "touched_experts_avg": round(avg["touched"], 2),
                   "step_hbm_gbs": round(step_gbs, 1),
                   "step_roofline_frac": round(step_gbs / HBM_PEAK_GBS, 4)},
        "roofline": roof,
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline(wl, args),
    }
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


def cpu_baseline(wl, args):
    """The oracle as it stands, on the host cores, on a bounded sample."""
    import synth
    from oracle import Oracle, Weights
    threads = min(16, os.cpu_count() or 1)
    orc = Oracle()
    if wl.name == "decode_t1":
        L = synth.make_layer(wl.name, T=max(1, threads * 2))
        n = L.wl.T
        tokens = None
        sample = f"{n} single-token decode forwards (router on x), all layer shapes as timed"
    else:
        L = synth.make_layer(wl.name)
        n = min(wl.T, max(threads * 2, 8))
        tokens = list(range(0, wl.T, max(1, wl.T // n)))[:n]
        sample = f"{len(tokens)} of the {wl.T} tokens of the timed batch (same weights and routing)"
    W = Weights.from_layer(L)
    t0 = time.perf_counter()
    orc.forward(W, L.wr, L.x, L.wl.k, ids=L.ids, w=L.w, tokens=tokens, threads=threads)
    el = time.perf_counter() - t0
    ntok = n if tokens is None else len(tokens)
    return {"value": round(ntok / el, 4), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": sample, "seconds": round(el, 2)}


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
    ap.add_argument("--calib-mib", type=int, default=0,
                    help="after timing, run a plain float32 add of this many MiB (counter calibration)")
    ap.add_argument("--summarize", default=None)
    ap.add_argument("--kind", default="trace")
    ap.add_argument("--command", default="")
    args = ap.parse_args()
    if args.summarize:
        return summarize(args)
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
