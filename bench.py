#!/usr/bin/env python3
"""Benchmark of the fused MoE forward on one MI355X.

One step = one moe_forward (sort, GEMM1 + SwiGLU, GEMM2, finalize) over one
batch of seeded synthetic inputs already resident in HBM.  The headline
workload is W4A16 decode (M=8 tokens, hidden 6144, inter 2048, 256 experts
of which 32 are local, top_k 8), HBM-bound on weight bytes; the W4A16
prefill workload (M=4096, biased router, SwiGLU limit 7), MFMA-bound, is
reported alongside in the same line, and so are the W4A4 (M=512) and
MXFP8 x MXFP4 (M=65536) parity configurations.  Weights, activations and routing are
rotated over several resident copies so that no step finds the previous
steps' weights in the 256 MB MALL.

Prints ONE JSON line (rank 0, N=1).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0       # dense fp8 MFMA
METRIC = "fused-MoE fwd tokens/s + % HBM roofline (M=8) / % MFMA peak (M=4096)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ inputs
class GpuInputs:
    """One workload's inputs on the GPU, prepared with the library's own
    quantisers from the seeded bf16 draws, in `copies` resident copies.
    W4A16: NVFP4 weights, bf16 x.  W4A4: NVFP4 weights and x (x's global
    scale folded into w1_alpha); fc2_input_scale is 1 (not calibrated: these
    inputs are for timing).  MXFP8_MXFP4: MXFP4 weights, MXFP8 x."""

    def __init__(self, wl, copies: int):
        import torch

        import mixture_experts_forward_moe_amd as moe
        import synth
        self.wl = wl
        E, H, I, M = wl.num_local_experts, wl.H, wl.I, wl.M
        R1 = I if wl.activation == 2 else 2 * I   # W1 rows: ReLU^2 is non-gated
        raw = synth.make_raw(wl)
        self.topk_ids_np = raw.topk_ids
        dev = "cuda"
        xb = torch.from_numpy(raw.x.view(np.int16)).to(dev)
        w1b = torch.from_numpy(raw.w1.view(np.int16)).to(dev)
        w2b = torch.from_numpy(raw.w2.view(np.int16)).to(dev)
        del raw
        u8 = dict(dtype=torch.uint8, device=dev)
        self.x_sf = None
        self.fc2 = None
        if wl.mode == moe.MXFP8_MXFP4:
            self.w1 = torch.empty((E, R1, H // 2), **u8)
            self.w1_sf = torch.empty((E, R1, H // 32), **u8)
            self.w2 = torch.empty((E, H, I // 2), **u8)
            self.w2_sf = torch.empty((E, H, I // 32), **u8)
            moe.moe_quantize_mx(w1b, E * R1, H, 1, self.w1, self.w1_sf)
            moe.moe_quantize_mx(w2b, E * H, I, 1, self.w2, self.w2_sf)
            self.w1_alpha = torch.ones(E, dtype=torch.float32, device=dev)
            self.w2_alpha = torch.ones(E, dtype=torch.float32, device=dev)
            self.x = torch.empty((M, H), **u8)
            self.x_sf = torch.empty((M, H // 32), **u8)
            moe.moe_quantize_mx(xb, M, H, 0, self.x, self.x_sf)
        else:
            self.w1 = torch.empty((E, R1, H // 2), **u8)
            self.w1_sf = torch.empty((E, R1, H // 16), **u8)
            self.w2 = torch.empty((E, H, I // 2), **u8)
            self.w2_sf = torch.empty((E, H, I // 16), **u8)
            self.w1_alpha = torch.empty(E, dtype=torch.float32, device=dev)
            self.w2_alpha = torch.empty(E, dtype=torch.float32, device=dev)
            moe.moe_nvfp4_global_scale(w1b, E, self.w1_alpha)
            moe.moe_quantize_nvfp4(w1b, E, R1, H, self.w1_alpha, self.w1, self.w1_sf)
            moe.moe_nvfp4_global_scale(w2b, E, self.w2_alpha)
            moe.moe_quantize_nvfp4(w2b, E, H, I, self.w2_alpha, self.w2, self.w2_sf)
            if wl.mode == moe.W4A4:
                xg = torch.empty(1, dtype=torch.float32, device=dev)
                moe.moe_nvfp4_global_scale(xb, 1, xg)
                self.x = torch.empty((M, H // 2), **u8)
                self.x_sf = torch.empty((M, H // 16), **u8)
                moe.moe_quantize_nvfp4(xb, 1, M, H, xg, self.x, self.x_sf)
                self.w1_alpha *= xg
                self.fc2 = torch.ones(1, dtype=torch.float32, device=dev)
            else:
                self.x = xb
        torch.cuda.synchronize()
        del w1b, w2b
        self.ids = torch.from_numpy(self.topk_ids_np).to(dev)
        _, wts = synth.make_routing(wl)
        self.w = torch.from_numpy(wts).to(dev)
        # resident copies, rotated step by step
        self.copies = [(self.x, self.ids, self.w, self.w1, self.w1_sf, self.w1_alpha, self.w2, self.w2_sf,
                        self.w2_alpha, self.x_sf)]
        for _ in range(copies - 1):
            self.copies.append(tuple(t.clone() if t is not None else None for t in self.copies[0]))
        torch.cuda.synchronize()

    def local_stats(self):
        wl = self.wl
        ids = self.topk_ids_np
        local = (ids >= wl.local_expert_offset) & (ids < wl.local_expert_offset + wl.num_local_experts)
        routes = int(local.sum())
        active = int(np.unique(ids[local]).size)
        return routes, active


def _opts(moe, wl, ws, tile, fc2=None, **kw):
    return moe.make_opts(workspace=ws, tile=tile, swiglu_alpha=wl.swiglu_alpha, swiglu_beta=wl.swiglu_beta,
                         swiglu_limit=wl.swiglu_limit, activation=wl.activation, situ_beta=wl.situ_beta,
                         situ_linear_beta=wl.situ_linear_beta, fc2_input_scale=fc2, **kw)


def _scale_kw(g, scaled: bool):
    """Options of the scaled variant: the up half with its own per-expert
    scale (1.5x the gate's), FC1 and FC2 biases (0.01) and
    routed_scaling_factor 1.75."""
    if not scaled:
        return {}
    import torch
    w1a = g.copies[0][5]
    E, H, I = g.wl.num_local_experts, g.wl.H, g.wl.I
    return dict(w1_alpha_up=(w1a * 1.5).contiguous(), routed_scaling_factor=1.75,
                fc1_bias=torch.full((E, 2 * I), 0.01, dtype=torch.float32, device="cuda"),
                fc2_bias=torch.full((E, H), 0.01, dtype=torch.float32, device="cuda"))


def time_graph(wl, steps: int, warmup: int, copies: int, scaled: bool = False):
    """Times `steps` forwards replayed from a HIP graph that holds `copies`
    forwards, one per resident input copy (no host work between launches).
    HIP events on the replay stream bracket the timed replays."""
    import torch

    import mixture_experts_forward_moe_amd as moe
    g = GpuInputs(wl, copies)
    H, I, E = wl.H, wl.I, wl.num_local_experts
    tile = moe.default_tile(wl.M, wl.top_k, wl.num_experts, E, wl.mode)
    ws = torch.zeros(moe.workspace_size(wl.M, H, I, wl.top_k, E, tile, wl.mode), dtype=torch.uint8, device="cuda")
    out = torch.empty((wl.M, H), dtype=torch.int16, device="cuda")
    skw = _scale_kw(g, scaled)
    opts = _opts(moe, wl, ws, tile, fc2=g.fc2, **skw)

    def step(i):
        x, ids, w, w1, w1s, w1a, w2, w2s, w2a, xs = g.copies[i % len(g.copies)]
        moe.moe_forward(x, xs, ids, w, w1, w1s, w1a, w2, w2s, w2a, wl.num_experts, wl.top_k, E,
                        wl.local_expert_offset, wl.mode, out, H, I, opts=opts)

    for i in range(max(warmup, copies)):  # eager warm-up (also caches the launch shape)
        step(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(copies):
            step(i)
    reps = max(1, steps // copies)
    for _ in range(max(1, warmup // copies)):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    n = reps * copies
    gpu_ms = e0.elapsed_time(e1)
    routes, active = g.local_stats()
    del graph, g
    torch.cuda.empty_cache()
    return dict(steps=n, seconds=dt, ms_per_step=dt * 1e3 / n, gpu_ms_per_step=gpu_ms / n, tile=tile,
                local_routes=routes, active_experts=active)


def time_phases(wl, steps: int, warmup: int, copies: int, scaled: bool = False):
    """Times `steps` eager forwards, then the same steps again with HIP
    events that moe_forward records between its launches on the same
    stream (per-kernel durations)."""
    import torch

    import mixture_experts_forward_moe_amd as moe
    g = GpuInputs(wl, copies)
    H, I, E = wl.H, wl.I, wl.num_local_experts
    tile = moe.default_tile(wl.M, wl.top_k, wl.num_experts, E, wl.mode)
    ws = torch.zeros(moe.workspace_size(wl.M, H, I, wl.top_k, E, tile, wl.mode), dtype=torch.uint8, device="cuda")
    out = torch.empty((wl.M, H), dtype=torch.int16, device="cuda")
    nev = moe.NUM_PHASE_EVENTS
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(steps)]
    for row in events:          # torch creates an event on its first record
        for e in row:
            e.record()
    torch.cuda.synchronize()
    skw = _scale_kw(g, scaled)
    opts = _opts(moe, wl, ws, tile, fc2=g.fc2, **skw)
    opts_ev = [_opts(moe, wl, ws, tile, fc2=g.fc2, phase_events=events[i], **skw) for i in range(steps)]

    def step(i, o):
        x, ids, w, w1, w1s, w1a, w2, w2s, w2a, xs = g.copies[i % len(g.copies)]
        moe.moe_forward(x, xs, ids, w, w1, w1s, w1a, w2, w2s, w2a, wl.num_experts, wl.top_k, E,
                        wl.local_expert_offset, wl.mode, out, H, I, opts=o)

    for i in range(warmup):
        step(i, opts)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i, opts)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    for i in range(steps):
        step(i, opts_ev[i])
    torch.cuda.synchronize()
    names = ["sort", "gemm1", "gemm2", "finalize"]
    per = {n: float(np.mean([events[i][k].elapsed_time(events[i][k + 1]) for i in range(steps)]))
           for k, n in enumerate(names)}
    routes, active = g.local_stats()
    del g
    torch.cuda.empty_cache()
    return dict(steps=steps, seconds=dt, ms_per_step=dt * 1e3 / steps, tile=tile, phase_ms=per,
                local_routes=routes, active_experts=active)


# ------------------------------------------------------------------ algorithmic work
def w4a16_bytes(wl, routes, active):
    """Algorithmic HBM bytes: active experts' NVFP4 weights (codes + E4M3
    block scales); per local route its token's bf16 row read, y1 written and
    read, y2 written and read; routing ids and weights read; the output
    written once."""
    H, I = wl.H, wl.I
    R1 = I if wl.activation == 2 else 2 * I   # W1 rows: ReLU^2 is non-gated
    w1 = R1 * H // 2 + R1 * H // 16
    w2 = H * I // 2 + H * I // 16
    act = routes * (2 * H + 2 * 2 * I + 2 * 2 * H)
    io = wl.M * wl.top_k * 8 + wl.M * H * 2
    return dict(
        gemm1=active * w1 + routes * (H * 2 + I * 2),
        gemm2=active * w2 + routes * (I * 2 + H * 2),
        forward=active * (w1 + w2) + act + io,
        weights=active * (w1 + w2),
        w1_per_expert=w1, w2_per_expert=w2,
    )


def weight_bytes(wl, active):
    """Codes and block scales of the active experts' W1 and W2 (NVFP4:
    E4M3 per 16 elements; MXFP4: E8M0 per 32)."""
    import synth
    blk = 32 if wl.mode == synth.MXFP8_MXFP4 else 16
    per = 3 * wl.H * wl.I // 2 + 3 * wl.H * wl.I // blk
    return active * per


def flops(wl, routes):
    return 6.0 * wl.H * wl.I * routes


# ------------------------------------------------------------------ measured traffic
def counter_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE record of this kernel and workload, scaled by the copy
    calibration; None when there is no record or the kernel source has
    changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = os.path.join(ROOT, rec["source"])
    if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != rec["source_sha256"]:
        return None
    return rec["traffic_bytes_per_launch"]


# ------------------------------------------------------------------ cpu baseline
def cpu_baseline(wl, min_seconds=10.0):
    """The oracle as it stands, on the host cores, over every token of the
    workload (repeated until ~min_seconds of CPU work)."""
    import oracle
    import synth
    p = oracle.quantize_problem(synth.make_raw(wl))
    toks = np.arange(wl.M, dtype=np.int32)
    n = 0
    t0 = time.perf_counter()
    while True:
        oracle.forward_tokens(p, toks)
        n += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = time.perf_counter() - t0
    return dict(value=wl.M * n / dt, unit="tokens/s", cores=oracle.num_threads(), kind="oracle",
                sample=f"all {wl.M} tokens of {wl.name}, {n} pass(es) in {dt:.1f} s (fp64 C oracle, OpenMP)")


# ------------------------------------------------------------------ counter calibration
def copy_calibration(steps: int, nbytes: int = 1 << 28):
    """A plain device-to-device copy of nbytes, `steps` times: its
    FETCH_SIZE / WRITE_SIZE per dispatch against nbytes gives the factor
    that turns those counters into HBM bytes."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    print(json.dumps({"copy_bytes": nbytes, "read_bytes": nbytes, "write_bytes": nbytes, "steps": steps,
                      "ms_per_copy": ms, "GBps_read_plus_write": 2 * nbytes / (ms * 1e-3) / 1e9}), flush=True)


# ------------------------------------------------------------------ main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=6, help="resident input copies rotated over steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--workload", default="w4a16_decode")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (scales the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only (the expert-parallel sharding across GPUs is a design, "
              "not code); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        copy_calibration(args.steps)
        return
    import mixture_experts_forward_moe_amd as moe
    import synth
    moe.lib()  # fail loudly if the native library is missing
    assert torch.cuda.is_available(), "no GPU"
    wl = synth.WORKLOADS[args.workload]

    log(f"bench: {wl.name}: {args.steps} steps after {args.warmup} warm-up (graph replay)")
    r = time_graph(wl, args.steps, args.warmup, args.copies)
    routes, active = r["local_routes"], r["active_experts"]
    by = w4a16_bytes(wl, routes, active)
    fl = flops(wl, routes)
    tokens_s = wl.M * r["steps"] / r["seconds"]
    # The decode forward is two launches (dec_gemm1_kernel with the routing
    # plan, dec_gemm2_kernel with the finalize) replayed back to back from a
    # HIP graph; the roofline takes the pair as its unit: algorithmic bytes
    # of the forward over the forward's time from HIP events around the
    # replays.  Per-kernel times come from eager steps with HIP events
    # recorded between the two launches (they include the event's own
    # dispatch gap, a few microseconds per kernel).
    log(f"bench: {wl.name}: {args.steps} eager steps with per-kernel events")
    rk = time_phases(wl, args.steps, args.warmup, args.copies)
    k1_ms, k2_ms = rk["phase_ms"]["gemm1"], rk["phase_ms"]["gemm2"]
    f_ms = r["gpu_ms_per_step"]
    f_gbs = by["forward"] / (f_ms * 1e-3) / 1e9
    w_gbs = by["weights"] / (f_ms * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": tokens_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": r["steps"],
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "quant_mode": "w4a16 (NVFP4 weights, bf16 activations)", "M": wl.M,
                   "H": wl.H, "I": wl.I, "num_experts": wl.num_experts, "num_local_experts": wl.num_local_experts,
                   "top_k": wl.top_k, "tile": r["tile"], "finalize": "deterministic", "local_routes": routes,
                   "active_local_experts": active, "resident_copies": args.copies, "launch": "hip graph replay"},
        "roofline": {"bound": "hbm", "kernel": "dec_gemm1_kernel + dec_gemm2_kernel (one decode forward)",
                     "achieved": f_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": f_gbs / HBM_PEAK_GBS,
                     "traffic": counter_traffic("dec_forward", wl.name),
                     "algorithmic_bytes": by["forward"], "avg_ms": f_ms},
        "kernels": {"dec_gemm1_kernel": {"avg_ms": k1_ms, "algorithmic_bytes": by["gemm1"],
                                         "GBps": by["gemm1"] / (k1_ms * 1e-3) / 1e9},
                    "dec_gemm2_kernel": {"avg_ms": k2_ms, "algorithmic_bytes": by["gemm2"],
                                         "GBps": by["gemm2"] / (k2_ms * 1e-3) / 1e9,
                                         "note": "includes the route-order finalize of its last workgroups"},
                    "timing": "eager steps, HIP events between the launches"},
        "weights": {"bytes": by["weights"], "GBps": w_gbs, "hbm_frac": w_gbs / HBM_PEAK_GBS,
                    "tflops": fl / (f_ms * 1e-3) / 1e12},
    }
    if not args.no_secondary:
        wl2 = synth.WORKLOADS["w4a16_prefill"]
        steps2 = max(10, args.steps // 10)
        log(f"bench: {wl2.name}: {steps2} steps (eager, per-kernel events)")
        r2 = time_phases(wl2, steps2, max(3, args.warmup // 4), args.copies)
        fl2 = flops(wl2, r2["local_routes"])
        tf2 = fl2 / (r2["ms_per_step"] * 1e-3) / 1e12
        g1f = 4.0 * wl2.H * wl2.I * r2["local_routes"] / (r2["phase_ms"]["gemm1"] * 1e-3) / 1e12
        line["prefill"] = {"workload": wl2.name, "M": wl2.M, "tokens_per_s": wl2.M * steps2 / r2["seconds"],
                           "ms_per_step": r2["ms_per_step"], "tile": r2["tile"], "local_routes": r2["local_routes"],
                           "tflops": tf2, "mfma_frac": tf2 / BF16_PEAK_TFLOPS, "gemm1_tflops": g1f,
                           "gemm1_mfma_frac": g1f / BF16_PEAK_TFLOPS, "phase_ms": r2["phase_ms"],
                           "peak_tflops": BF16_PEAK_TFLOPS}
    if not args.no_secondary:
        # the other two quantisation modes, on their parity configurations
        for name, key, peak, steps3, note in (
                ("w4a4", "w4a4_nvfp4", BF16_PEAK_TFLOPS, 10, "NVFP4 x and weights, bf16 MFMA after decode"),
                ("mx", "mxfp8_mxfp4_large", FP8_PEAK_TFLOPS, 4,
                 "MXFP8 x, MXFP4 weights, scaled fp8 x fp4 MFMA (peak: dense fp8)")):
            wl3 = synth.WORKLOADS[key]
            log(f"bench: {wl3.name}: {steps3} steps (eager, per-kernel events)")
            r3 = time_phases(wl3, steps3, 2, 1)
            fl3 = flops(wl3, r3["local_routes"])
            tf3 = fl3 / (r3["ms_per_step"] * 1e-3) / 1e12
            wb = weight_bytes(wl3, r3["active_experts"])
            line[name] = {"workload": wl3.name, "M": wl3.M, "H": wl3.H, "I": wl3.I,
                          "local_experts": wl3.num_local_experts, "tokens_per_s": wl3.M * steps3 / r3["seconds"],
                          "ms_per_step": r3["ms_per_step"], "tile": r3["tile"], "local_routes": r3["local_routes"],
                          "tflops": tf3, "mfma_frac": tf3 / peak, "peak_tflops": peak, "phase_ms": r3["phase_ms"],
                          "weight_bytes": wb, "weights_hbm_frac": wb / (r3["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                          "note": note}
    if not args.no_secondary:
        # the other GEMM epilogues on the decode and prefill workloads (GeGLU-tanh, SiTU, and SwiGLU with
        # the up half's own scale, FC1 / FC2 biases and routed_scaling_factor 1.75): the decode forward in graph replay
        # (same roofline unit as the headline) and the prefill GEMM1 with per-kernel events
        import dataclasses
        acts = {}
        for name, kw in (("geglu_tanh", dict(activation=1)), ("situ", dict(situ_beta=0.5, situ_linear_beta=1.0)),
                         ("relu2", dict(activation=2)), ("swiglu_scaled", dict())):
            scaled = name == "swiglu_scaled"
            wd = dataclasses.replace(wl, **kw)
            log(f"bench: {wd.name} with {name}: {max(20, args.steps // 4)} steps (graph replay)")
            rd = time_graph(wd, max(20, args.steps // 4), max(4, args.warmup // 4), args.copies, scaled=scaled)
            fd = w4a16_bytes(wd, routes, active)["forward"] / (rd["gpu_ms_per_step"] * 1e-3) / 1e9
            wp = dataclasses.replace(synth.WORKLOADS["w4a16_prefill"], swiglu_limit=float(np.finfo(np.float32).max),
                                     **kw)
            rp = time_phases(wp, 10, 3, args.copies, scaled=scaled)
            g1 = (2.0 if wp.activation == 2 else 4.0) * wp.H * wp.I * rp["local_routes"] / (
                rp["phase_ms"]["gemm1"] * 1e-3) / 1e12
            if scaled:
                kw = {"w1_alpha_up": "1.5 x w1_alpha", "fc1_bias": 0.01, "fc2_bias": 0.01,
                      "routed_scaling_factor": 1.75}
            acts[name] = {"params": kw, "decode_ms_per_forward": rd["gpu_ms_per_step"], "decode_hbm_frac": fd / HBM_PEAK_GBS,
                          "prefill_gemm1_ms": rp["phase_ms"]["gemm1"], "prefill_gemm1_mfma_frac": g1 / BF16_PEAK_TFLOPS}
        acts["swiglu"] = {"decode_ms_per_forward": f_ms, "decode_hbm_frac": f_gbs / HBM_PEAK_GBS,
                          "prefill_gemm1_ms": line["prefill"]["phase_ms"]["gemm1"],
                          "prefill_gemm1_mfma_frac": line["prefill"]["gemm1_mfma_frac"],
                          "note": "prefill with SwiGLU limit 7 (its workload); the others without a limit"}
        line["epilogue_variants"] = acts
    if not args.no_cpu_baseline:
        log("bench: CPU oracle baseline")
        line["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
