#!/usr/bin/env python3
"""Benchmark of the fused MoE forward on one MI355X.

One step = one moe_forward (sort, GEMM1 + SwiGLU, GEMM2, finalize) over one
batch of seeded synthetic inputs already resident in HBM.  The headline
workload is W4A16 decode (M=8 tokens, hidden 6144, inter 2048, 256 experts
of which 32 are local, top_k 8), HBM-bound on weight bytes; the W4A16
prefill workload (M=4096, biased router, SwiGLU limit 7), MFMA-bound, is
reported alongside in the same line, and so are the W4A4 (M=512, with a
calibrated fc2_input_scale) and MXFP8 x MXFP4 (M=65536) configurations.
Weights, activations and routing are rotated over several resident copies
so that no step finds the previous steps' weights in the 256 MB MALL (the
"cold" figure, the metric); the "warm" figure replays one copy.

The headline decode forward uses the fused finalize (GEMM2 adds each
route's scaled rows into the output with packed-bf16 atomics), the
default of the pages' API ("flashinfer.fused_moe.cute_dsl_fused_moe",
Parameters: use_fused_finalize); the same forward with the deterministic
route-order finalize is reported beside it.

Also in the line: per-forward latency percentiles, the measured streaming
copy bandwidth as a second roofline denominator, the routing-locality
report of the large-batch plan (distinct 2 MiB pages of x per GEMM1 tile)
and the CPU oracle timed on the host cores.

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


def pct(v):
    """median, p10, p90 of a list of times (ms)"""
    a = np.asarray(v, np.float64)
    return {"median_ms": float(np.median(a)), "p10_ms": float(np.percentile(a, 10)),
            "p90_ms": float(np.percentile(a, 90)), "samples": int(a.size)}


# ------------------------------------------------------------------ inputs
class GpuInputs:
    """One workload's inputs on the GPU, prepared with the library's own
    quantisers from the seeded bf16 draws, in `copies` resident copies.
    W4A16: NVFP4 weights, bf16 x.  W4A4: NVFP4 weights and x (x's global
    scale folded into w1_alpha) and fc2_input_scale calibrated on the device
    (moe_fc2_input_scale over the batch's routes, folded into w2_alpha).
    MXFP8_MXFP4: MXFP4 weights, MXFP8 x."""

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
        self.ids = torch.from_numpy(self.topk_ids_np).to(dev)
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
                # calibration pass on the device: max |y1| / (6 * 448) over the batch's routes
                tile = moe.default_tile(M, wl.top_k, wl.num_experts, E, wl.mode)
                plan = moe.moe_sort(self.ids, wl.num_experts, E, wl.local_expert_offset, tile)
                self.fc2 = torch.empty(1, dtype=torch.float32, device=dev)
                moe.moe_fc2_input_scale(self.x, self.x_sf, plan, self.w1, self.w1_sf, self.w1_alpha, H, I, self.fc2,
                                        activation=wl.activation, swiglu_alpha=wl.swiglu_alpha,
                                        swiglu_beta=wl.swiglu_beta, swiglu_limit=wl.swiglu_limit,
                                        situ_beta=wl.situ_beta, situ_linear_beta=wl.situ_linear_beta)
                self.w2_alpha *= self.fc2
                torch.cuda.synchronize()
                self.fc2_value = float(self.fc2.cpu()[0])
            else:
                self.x = xb
        torch.cuda.synchronize()
        del w1b, w2b
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


def _forwarder(moe, g, wl, out, opts):
    E, H, I = wl.num_local_experts, wl.H, wl.I

    def step(i):
        x, ids, w, w1, w1s, w1a, w2, w2s, w2a, xs = g.copies[i % len(g.copies)]
        moe.moe_forward(x, xs, ids, w, w1, w1s, w1a, w2, w2s, w2a, wl.num_experts, wl.top_k, E,
                        wl.local_expert_offset, wl.mode, out, H, I, opts=opts)
    return step


def time_graph(wl, steps: int, warmup: int, copies: int, scaled: bool = False, latency: int = 0,
               finalize_mode: int = 0):
    """Times `steps` forwards replayed from a HIP graph that holds `copies`
    forwards, one per resident input copy (no host work between launches).
    HIP events on the replay stream bracket the timed replays.  With
    latency > 0, also per-forward times: one graph per copy, `latency`
    replays rotating over the copies (cold) and on one copy (warm), an event
    between consecutive replays.  finalize_mode: moe.FINALIZE_* of the
    forwards."""
    import torch

    import mixture_experts_forward_moe_amd as moe
    g = GpuInputs(wl, copies)
    H, I, E = wl.H, wl.I, wl.num_local_experts
    tile = moe.default_tile(wl.M, wl.top_k, wl.num_experts, E, wl.mode)
    ws = torch.empty(moe.workspace_size(wl.M, H, I, wl.top_k, E, tile, wl.mode), dtype=torch.uint8, device="cuda")
    out = torch.empty((wl.M, H), dtype=torch.int16, device="cuda")
    skw = _scale_kw(g, scaled)
    opts = _opts(moe, wl, ws, tile, fc2=g.fc2, finalize_mode=finalize_mode, **skw)
    step = _forwarder(moe, g, wl, out, opts)

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
    res = dict(steps=n, seconds=dt, ms_per_step=dt * 1e3 / n, gpu_ms_per_step=gpu_ms / n, tile=tile)
    del graph
    if latency:
        singles = []
        for i in range(copies):
            gi = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gi):
                step(i)
            singles.append(gi)
        for which, order in (("cold", [i % copies for i in range(latency)]), ("warm", [0] * latency)):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(latency + 1)]
            for i in range(copies):
                singles[i].replay()
            torch.cuda.synchronize()
            ev[0].record()
            for i, c in enumerate(order):
                singles[c].replay()
                ev[i + 1].record()
            torch.cuda.synchronize()
            res[which] = pct([ev[i].elapsed_time(ev[i + 1]) for i in range(latency)])
        del singles
    res["local_routes"], res["active_experts"] = g.local_stats()
    del g
    torch.cuda.empty_cache()
    return res


def time_phases(wl, steps: int, warmup: int, copies: int, scaled: bool = False, plan_out: dict | None = None,
                finalize_mode: int = 0):
    """Times `steps` eager forwards, then the same steps again with HIP
    events that moe_forward records between its launches on the same
    stream (per-kernel durations, and per-step forward times for the
    percentiles)."""
    import torch

    import mixture_experts_forward_moe_amd as moe
    g = GpuInputs(wl, copies)
    H, I, E = wl.H, wl.I, wl.num_local_experts
    tile = moe.default_tile(wl.M, wl.top_k, wl.num_experts, E, wl.mode)
    ws = torch.empty(moe.workspace_size(wl.M, H, I, wl.top_k, E, tile, wl.mode), dtype=torch.uint8, device="cuda")
    out = torch.empty((wl.M, H), dtype=torch.int16, device="cuda")
    nev = moe.NUM_PHASE_EVENTS
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(steps)]
    for row in events:          # torch creates an event on its first record
        for e in row:
            e.record()
    torch.cuda.synchronize()
    skw = _scale_kw(g, scaled)
    opts = _opts(moe, wl, ws, tile, fc2=g.fc2, finalize_mode=finalize_mode, **skw)
    opts_ev = [_opts(moe, wl, ws, tile, fc2=g.fc2, phase_events=events[i], finalize_mode=finalize_mode, **skw)
               for i in range(steps)]
    step = _forwarder(moe, g, wl, out, opts)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    for i in range(steps):
        _forwarder(moe, g, wl, out, opts_ev[i])(i)
    torch.cuda.synchronize()
    names = ["sort", "gemm1", "gemm2", "finalize"]
    per = {n: float(np.mean([events[i][k].elapsed_time(events[i][k + 1]) for i in range(steps)]))
           for k, n in enumerate(names)}
    fwd = pct([events[i][0].elapsed_time(events[i][nev - 1]) for i in range(steps)])
    routes, active = g.local_stats()
    if plan_out is not None:
        # the plan this forward used, read back from its workspace
        p = moe.MoePlan(wl.M, wl.top_k, E, tile, forward_workspace=ws)
        plan_out.update(tile=tile, p2e=p.permuted_to_expanded.cpu().numpy(),
                        tile_expert=p.tile_to_expert.cpu().numpy(), tile_limit=p.tile_to_mn_limit.cpu().numpy(),
                        num_tiles=int(p.num_tiles.cpu()[0]))
    res = dict(steps=steps, seconds=dt, ms_per_step=dt * 1e3 / steps, tile=tile, phase_ms=per, forward=fwd,
               local_routes=routes, active_experts=active, fc2_input_scale=getattr(g, "fc2_value", None))
    del g
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------ algorithmic work
def w4a16_bytes(wl, routes, active, atomic: bool = False):
    """Algorithmic HBM bytes: active experts' NVFP4 weights (codes + E4M3
    block scales); per local route its token's bf16 row read, y1 written and
    read, and y2 written and read (deterministic finalize) or its row added
    into the output once (atomic finalize, after GEMM1 has zeroed the
    output); routing ids and weights read; the output written once."""
    H, I = wl.H, wl.I
    R1 = I if wl.activation == 2 else 2 * I   # W1 rows: ReLU^2 is non-gated
    w1 = R1 * H // 2 + R1 * H // 16
    w2 = H * I // 2 + H * I // 16
    y2 = 2 * H if atomic else 2 * 2 * H
    act = routes * (2 * H + 2 * 2 * I + y2)
    io = wl.M * wl.top_k * 8 + wl.M * H * 2
    return dict(
        gemm1=active * w1 + routes * (H * 2 + I * 2) + (wl.M * H * 2 if atomic else 0),
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
def counter_traffic(kernel: str, workload: str, finalize: str | None = None):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE record of this kernel and workload (and finalize mode, where
    the record names one), scaled by the copy calibration; None when there
    is no record, it was taken in another finalize mode, or the kernel
    source has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if finalize is not None and rec.get("finalize", "deterministic") != finalize:
        return None
    src = os.path.join(ROOT, rec["source"])
    if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != rec["source_sha256"]:
        return None
    return rec["traffic_bytes_per_launch"]


# ------------------------------------------------------------------ routing locality
def locality_report(plan: dict, wl, tiles=(128, 256), seed: int = 4):
    """Distinct 2 MiB pages of x a GEMM1 tile gathers from (MXFP8 x rows of
    H bytes), computed on the host from the plan the forward used: for its
    stable route order, and for a simulated grid-stride arrival order (each
    of G = 256 workgroups x 1024 threads takes routes t, t + G, ...; inside
    one stride the arrival order is a seeded random permutation) at the same
    per-expert tile padding.  Tiles of 128 slots (this build's) and of 256
    (the pages' large-batch tile) are both counted."""
    k, H = wl.top_k, wl.H
    page = 2 << 20
    p2e = plan["p2e"]
    nt, T0 = plan["num_tiles"], plan["tile"]
    by_expert = {}
    for i in range(nt):  # each expert's rows in the plan's (stable) order
        by_expert.setdefault(int(plan["tile_expert"][i]), []).append(p2e[i * T0:plan["tile_limit"][i]])
    experts = [np.concatenate(v).astype(np.int64) for v in by_expert.values()]
    assert sum(e.size for e in experts) == int((p2e >= 0).sum())
    G = 256 * 1024
    rng = np.random.default_rng(seed)
    R = wl.M * k
    rank = np.empty(R, np.int64)   # simulated arrival position of each route
    for s in range(0, R, G):
        rank[s:min(R, s + G)] = s + rng.permutation(min(R, s + G) - s)

    def pages_per_tile(order_rows, T):
        out = []
        for rows in order_rows:
            for i in range(0, rows.size, T):
                toks = rows[i:i + T] // k
                lo = (toks * H) // page
                hi = (toks * H + H - 1) // page
                out.append(np.unique(np.concatenate([lo, hi])).size)
        a = np.asarray(out)
        return {"mean": float(a.mean()), "median": float(np.median(a)), "max": int(a.max()), "tiles": int(a.size)}

    rep = {"unit": "distinct 2 MiB pages of x per GEMM1 tile", "x_row_bytes": H,
           "grid_stride_simulation": "G = 256 x 1024 threads, seeded random order within each stride"}
    for T in tiles:
        stable = pages_per_tile(experts, T)
        strided = pages_per_tile([e[np.argsort(rank[e], kind="stable")] for e in experts], T)
        rep[f"tile{T}"] = {"stable_order": stable, "grid_stride_order": strided}
    return rep


# ------------------------------------------------------------------ cpu baseline
def cpu_baseline(headline: str, min_seconds: float = 2.0):
    """The oracle as it stands, on the host cores: each workload's forward
    after its inputs are quantised (input preparation is not timed).  The
    decode and tiny workloads run all their tokens repeatedly for about
    min_seconds; prefill and W4A4 one plan-based pass over every token; the
    M = 65536 MX workload its routing plan for all tokens plus the per-token
    forward of its 1024 sampled tokens (a sampled rate)."""
    import oracle
    import synth
    per = {}
    for name, wl in synth.WORKLOADS.items():
        t_prep = time.perf_counter()
        p = oracle.quantize_problem(synth.make_raw(wl))
        prep = time.perf_counter() - t_prep
        ids = p.topk_ids
        local = (ids >= wl.local_expert_offset) & (ids < wl.local_expert_offset + wl.num_local_experts)
        if wl.sample_tokens:
            toks = synth.sample_tokens(wl.seed, wl.M, wl.sample_tokens)
            t0 = time.perf_counter()
            oracle.sort(ids, wl.num_local_experts, wl.local_expert_offset, 128)
            t_plan = time.perf_counter() - t0
            t0 = time.perf_counter()
            oracle.forward_tokens(p, toks)
            dt = time.perf_counter() - t0
            routes = int(local[toks].sum())
            per[name] = {"tokens_per_s": toks.size / dt, "gflops": flops(wl, routes) / dt / 1e9, "seconds": dt,
                         "plan_seconds": t_plan, "sample": f"plan of all {wl.M} tokens; forward of {toks.size} "
                         f"sampled tokens (sampled rate)", "prep_seconds": prep}
        elif wl.M <= 64:
            toks = np.arange(wl.M, dtype=np.int32)
            n, t0 = 0, time.perf_counter()
            while True:
                oracle.forward_tokens(p, toks)
                n += 1
                if time.perf_counter() - t0 >= min_seconds:
                    break
            dt = time.perf_counter() - t0
            per[name] = {"tokens_per_s": wl.M * n / dt, "gflops": n * flops(wl, int(local.sum())) / dt / 1e9,
                         "seconds": dt, "sample": f"all {wl.M} tokens, {n} pass(es)", "prep_seconds": prep}
        else:
            t0 = time.perf_counter()
            oracle.forward_plan(p, 64)
            dt = time.perf_counter() - t0
            per[name] = {"tokens_per_s": wl.M / dt, "gflops": flops(wl, int(local.sum())) / dt / 1e9,
                         "seconds": dt, "sample": f"all {wl.M} tokens, one plan-based pass", "prep_seconds": prep}
        log(f"bench: cpu oracle {name}: {per[name]['tokens_per_s']:.1f} tokens/s")
    h = per[headline]
    return dict(value=h["tokens_per_s"], unit="tokens/s", cores=oracle.num_threads(), kind="oracle",
                sample=f"{headline}: {h['sample']} ({h['seconds']:.1f} s, fp64 C oracle, OpenMP); every "
                       f"workload in per_config", gflops=h["gflops"], per_config=per)


# ------------------------------------------------------------------ copy bandwidth
def copy_bandwidth(nbytes: int = 1 << 30, reps: int = 20):
    """A plain device-to-device copy of nbytes: bytes read plus written per
    second (the streaming bandwidth this machine reaches; the second roofline
    denominator)."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes_copied": nbytes, "ms_per_copy": ms, "GBps": 2 * nbytes / (ms * 1e-3) / 1e9}


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
def secondary(name, wl, r, peak, copy_gbs, note):
    fl = flops(wl, r["local_routes"])
    ms = r["forward"]["median_ms"]
    tf = fl / (ms * 1e-3) / 1e12
    wb = weight_bytes(wl, r["active_experts"])
    d = {"workload": wl.name, "M": wl.M, "H": wl.H, "I": wl.I, "local_experts": wl.num_local_experts,
         "tokens_per_s": wl.M * r["steps"] / r["seconds"], "ms_per_step": r["ms_per_step"], "forward": r["forward"],
         "tile": r["tile"], "local_routes": r["local_routes"], "tflops": tf, "mfma_frac": tf / peak,
         "peak_tflops": peak, "phase_ms": r["phase_ms"], "weight_bytes": wb,
         "weights_GBps": wb / (ms * 1e-3) / 1e9, "weights_hbm_frac": wb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
         "weights_copy_frac": wb / (ms * 1e-3) / 1e9 / copy_gbs,
         "note": note + "; rates from the median per-step forward time (HIP events)"}
    g1f = (2.0 if wl.activation == 2 else 4.0) * wl.H * wl.I * r["local_routes"] / (
        r["phase_ms"]["gemm1"] * 1e-3) / 1e12
    d["gemm1_tflops"] = g1f
    d["gemm1_mfma_frac"] = g1f / peak
    if r.get("fc2_input_scale") is not None:
        d["fc2_input_scale"] = r["fc2_input_scale"]
    return d


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=6, help="resident input copies rotated over steps")
    ap.add_argument("--latency-samples", type=int, default=300, help="forwards timed one by one for percentiles")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--finalize", choices=["atomic", "deterministic"], default="atomic",
                    help="finalize of the headline decode forward (atomic: the pages' default)")
    ap.add_argument("--no-other-finalize", action="store_true",
                    help="skip the decode forward with the other finalize (for counter runs)")
    ap.add_argument("--workload", default="w4a16_decode")
    ap.add_argument("--only", choices=["prefill", "w4a4", "mx"], default=None,
                    help="profiling aid: time only this secondary workload (no headline line)")
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
    if args.only:
        key = {"prefill": "w4a16_prefill", "w4a4": "w4a4_nvfp4", "mx": "mxfp8_mxfp4_large"}[args.only]
        wo = synth.WORKLOADS[key]
        peak = FP8_PEAK_TFLOPS if args.only == "mx" else BF16_PEAK_TFLOPS
        steps = max(2, args.steps)
        log(f"bench: {wo.name} only: {steps} steps (eager, per-kernel events)")
        ro = time_phases(wo, steps, args.warmup, 1 if args.only == "mx" else args.copies)
        print(json.dumps({args.only: secondary(args.only, wo, ro, peak, float("nan"), "profiling run")}), flush=True)
        return

    log("bench: streaming copy bandwidth")
    cbw = copy_bandwidth()
    copy_gbs = cbw["GBps"]
    log(f"bench: {wl.name}: {args.steps} steps after {args.warmup} warm-up (graph replay), then "
        f"{args.latency_samples} forwards one by one")
    fmode = moe.FINALIZE_ATOMIC if args.finalize == "atomic" else moe.FINALIZE_DETERMINISTIC
    atomic = fmode == moe.FINALIZE_ATOMIC
    r = time_graph(wl, args.steps, args.warmup, args.copies, latency=args.latency_samples, finalize_mode=fmode)
    routes, active = r["local_routes"], r["active_experts"]
    by = w4a16_bytes(wl, routes, active, atomic=atomic)
    fl = flops(wl, routes)
    tokens_s = wl.M * r["steps"] / r["seconds"]
    # The decode forward is two launches (dec_gemm1_kernel with the routing
    # plan, dec_gemm2_kernel with the finalize: packed-bf16 atomics into the
    # output, or the route-order sums of its last workgroups) replayed back to back from a
    # HIP graph; the roofline takes the pair as its unit: algorithmic bytes
    # of the forward over the forward's time from HIP events around the
    # replays.  Per-kernel times come from eager steps with HIP events
    # recorded between the two launches (they include the event's own
    # dispatch gap, a few microseconds per kernel).
    log(f"bench: {wl.name}: {args.steps} eager steps with per-kernel events")
    rk = time_phases(wl, args.steps, args.warmup, args.copies, finalize_mode=fmode)
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
                   "top_k": wl.top_k, "tile": r["tile"], "finalize": args.finalize, "local_routes": routes,
                   "active_local_experts": active, "resident_copies": args.copies, "launch": "hip graph replay"},
        "roofline": {"bound": "hbm", "kernel": f"dec_gemm1_kernel + dec_gemm2_kernel<4, {str(atomic).lower()}> "
                                               "(one decode forward)",
                     "achieved": f_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": f_gbs / HBM_PEAK_GBS,
                     "traffic": counter_traffic("dec_forward", wl.name, args.finalize),
                     "algorithmic_bytes": by["forward"], "avg_ms": f_ms,
                     "copy_GBps": copy_gbs, "frac_of_copy": f_gbs / copy_gbs},
        "latency": {"cold": r["cold"], "warm": r["warm"],
                    "cold_hbm_frac": by["forward"] / (r["cold"]["median_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    "warm_hbm_frac": by["forward"] / (r["warm"]["median_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    "note": "per-forward times, one graph replay each: cold rotates the resident copies (no "
                            "MALL reuse), warm replays one copy (weights found in the 256 MB MALL)"},
        "copy_bandwidth": cbw,
        "kernels": {"dec_gemm1_kernel": {"avg_ms": k1_ms, "algorithmic_bytes": by["gemm1"],
                                         "GBps": by["gemm1"] / (k1_ms * 1e-3) / 1e9},
                    "dec_gemm2_kernel": {"avg_ms": k2_ms, "algorithmic_bytes": by["gemm2"],
                                         "GBps": by["gemm2"] / (k2_ms * 1e-3) / 1e9,
                                         "note": "includes the finalize: packed-bf16 atomics into out" if atomic
                                         else "includes the route-order finalize of its last workgroups"},
                    "timing": "eager steps, HIP events between the launches"},
        "weights": {"bytes": by["weights"], "GBps": w_gbs, "hbm_frac": w_gbs / HBM_PEAK_GBS,
                    "copy_frac": w_gbs / copy_gbs, "tflops": fl / (f_ms * 1e-3) / 1e12},
    }
    # the same decode forward with the other finalize: the deterministic
    # route-order sums (reproducible bit for bit) beside the atomic headline,
    # or the other way round
    if not args.no_other_finalize:
        other = "deterministic" if atomic else "atomic"
        log(f"bench: {wl.name}: {args.steps} steps with the {other} finalize (graph replay)")
        ro = time_graph(wl, args.steps, args.warmup, args.copies,
                        finalize_mode=moe.FINALIZE_DETERMINISTIC if atomic else moe.FINALIZE_ATOMIC)
        bo = w4a16_bytes(wl, routes, active, atomic=not atomic)["forward"]
        fo_gbs = bo / (ro["gpu_ms_per_step"] * 1e-3) / 1e9
        line["finalize_" + other] = {"tokens_per_s": wl.M * ro["steps"] / ro["seconds"],
                                     "ms_per_forward": ro["gpu_ms_per_step"], "GBps": fo_gbs,
                                     "hbm_frac": fo_gbs / HBM_PEAK_GBS, "copy_frac": fo_gbs / copy_gbs,
                                     "note": f"decode forward with the {other} finalize; the headline uses the "
                                             f"{args.finalize} one"}
    if not args.no_secondary:
        wl2 = synth.WORKLOADS["w4a16_prefill"]
        steps2 = max(20, args.steps // 10)
        log(f"bench: {wl2.name}: {steps2} steps (eager, per-kernel events)")
        r2 = time_phases(wl2, steps2, max(3, args.warmup // 4), args.copies)
        line["prefill"] = secondary("prefill", wl2, r2, BF16_PEAK_TFLOPS, copy_gbs, "W4A16, bf16 MFMA")
        for name, key, peak, steps3, copies3, note in (
                ("w4a4", "w4a4_nvfp4", BF16_PEAK_TFLOPS, 20, args.copies,
                 "NVFP4 x and weights, f16 MFMA after an exact decode of both; fc2_input_scale calibrated on the device"),
                ("mx", "mxfp8_mxfp4_large", FP8_PEAK_TFLOPS, 6, 1,
                 "MXFP8 x, MXFP4 weights, scaled fp8 x fp4 MFMA (peak: dense fp8)")):
            wl3 = synth.WORKLOADS[key]
            log(f"bench: {wl3.name}: {steps3} steps (eager, per-kernel events)")
            plan = {} if name == "mx" else None
            r3 = time_phases(wl3, steps3, 2, copies3, plan_out=plan)
            line[name] = secondary(name, wl3, r3, peak, copy_gbs, note)
            if plan:
                log("bench: routing locality of the large-batch plan")
                line[name]["locality"] = locality_report(plan, wl3)
    if not args.no_secondary and not args.no_variants:
        # the other GEMM epilogues on the decode and prefill workloads (GeGLU-tanh, SiTU, ReLU^2, and SwiGLU
        # with the up half's own scale, FC1 / FC2 biases and routed_scaling_factor 1.75): the decode
        # forward in graph replay (same roofline unit as the headline) and the prefill GEMM1 with per-kernel
        # events
        import dataclasses
        acts = {}
        for name, kw in (("geglu_tanh", dict(activation=1)), ("situ", dict(situ_beta=0.5, situ_linear_beta=1.0)),
                         ("relu2", dict(activation=2)), ("swiglu_scaled", dict())):
            scaled = name == "swiglu_scaled"
            wd = dataclasses.replace(wl, **kw)
            log(f"bench: {wd.name} with {name}: {max(20, args.steps // 4)} steps (graph replay)")
            rd = time_graph(wd, max(20, args.steps // 4), max(4, args.warmup // 4), args.copies, scaled=scaled,
                            finalize_mode=fmode)
            fd = w4a16_bytes(wd, routes, active, atomic=atomic)["forward"] / (rd["gpu_ms_per_step"] * 1e-3) / 1e9
            wp = dataclasses.replace(synth.WORKLOADS["w4a16_prefill"], swiglu_limit=float(np.finfo(np.float32).max),
                                     **kw)
            rp = time_phases(wp, 10, 3, args.copies, scaled=scaled)
            g1 = (2.0 if wp.activation == 2 else 4.0) * wp.H * wp.I * rp["local_routes"] / (
                rp["phase_ms"]["gemm1"] * 1e-3) / 1e12
            if scaled:
                kw = {"w1_alpha_up": "1.5 x w1_alpha", "fc1_bias": 0.01, "fc2_bias": 0.01,
                      "routed_scaling_factor": 1.75}
            acts[name] = {"params": kw, "decode_ms_per_forward": rd["gpu_ms_per_step"],
                          "decode_hbm_frac": fd / HBM_PEAK_GBS, "prefill_gemm1_ms": rp["phase_ms"]["gemm1"],
                          "prefill_gemm1_mfma_frac": g1 / BF16_PEAK_TFLOPS}
        acts["swiglu"] = {"decode_ms_per_forward": f_ms, "decode_hbm_frac": f_gbs / HBM_PEAK_GBS,
                          "prefill_gemm1_ms": line["prefill"]["phase_ms"]["gemm1"],
                          "prefill_gemm1_mfma_frac": line["prefill"]["gemm1_mfma_frac"],
                          "note": "prefill with SwiGLU limit 7 (its workload); the others without a limit"}
        line["epilogue_variants"] = acts
    if not args.no_cpu_baseline:
        log("bench: CPU oracle baseline")
        line["cpu_baseline"] = cpu_baseline(wl.name)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
