#!/usr/bin/env python
"""Benchmark of the FP4 routed-MoE layer on one MI355X.

The headline workload is the largest one that fits one GPU: 43 stacked MoE
layers with distinct weights (hidden 4096, intermediate 2048, 256 experts,
top-6, 147 GB resident), decode batch 32 with the residual stream
x <- x + moe_l(rmsnorm(x)), int8 activations. A step is one pass of that
batch through all 43 layers (route, sort, quantize, gate/up GEMM with
SiLU*mul, requantization, down GEMM, combine + residual + RMSNorm per layer).
The same workload's 16,384-token prefill chunk through one layer (MXFP4
activations, Zipf(1.1) expert load) gives the prefill FP4 roofline object;
the single-layer decode and prefill workloads are legs.

Prints one JSON line: tokens/s with the median and 10th/90th percentile of
the step times, the dominant kernel's roofline fraction (algorithmic bytes or
FLOPs per launch / its average duration from HIP events recorded on the
library's stream inside the timed region), the prefill gate/up kernel's FP4
fraction, a streaming-read ceiling, and the CPU oracle's tokens/s on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes as C
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP4_PEAK_TFLOPS = 10100.0       # MI355X dense MXFP4 MFMA, published
FP8_PEAK_TFLOPS = 5000.0        # MI355X dense FP8 MFMA, published
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")


# ----------------------------------------------------------------- HIP events
class HipEvents:
    # timing-only events: no system-scope fence (cache writeback/invalidate)
    # when they are recorded, so that they disturb the measured kernels less
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        self.hip = C.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [C.POINTER(C.c_void_p), C.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.hip.hipEventDestroy.argtypes = [C.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [C.c_void_p]

    def create(self, n):
        arr = (C.c_void_p * n)()
        for i in range(n):
            ev = C.c_void_p()
            assert self.hip.hipEventCreateWithFlags(C.byref(ev), self.DISABLE_SYSTEM_FENCE) == 0
            arr[i] = ev
        return arr

    def elapsed_ms(self, a, b) -> float:
        ms = C.c_float()
        assert self.hip.hipEventElapsedTime(C.byref(ms), a, b) == 0
        return ms.value

    def destroy(self, arr):
        for ev in arr:
            self.hip.hipEventDestroy(ev)


def per_expert_bytes(w):
    H, I = w.H, w.I
    w13 = 2 * I * H // 2 + 2 * I * H // 32
    w2 = H * I // 2 + H * I // 32
    return w13, w2


def layer_accounting(w, T: int, d_layer: float, d_gate_up: float, x_bf16: bool, int8: bool) -> dict:
    """Algorithmic work of one layer call on T tokens: the bytes the method
    must move (the weights, codes and scales, of the distinct routed experts
    d_layer, the router weights, x in and out) and its FP4 FLOPs (real pair
    rows only), plus the gate/up kernel's own bytes (the weights of the
    experts d_gate_up it streamed, quantized x in, its output) and FLOPs."""
    b13, b2 = per_expert_bytes(w)
    xbytes = T * w.H * (2 if x_bf16 else 4)
    P = T * w.top_k
    if int8:
        g1_bytes = d_gate_up * b13 + T * 2 * w.H + P * w.I * 4
    else:
        g1_bytes = d_gate_up * b13 + T * w.H // 2 + T * w.H // 32 + P * (w.I // 2 + w.I // 32)
    return {"layer_bytes": d_layer * (b13 + b2) + w.E * w.H * 4 + xbytes + T * w.H * 4,
            "layer_flops": 2.0 * P * (w.H * 2 * w.I + w.I * w.H),
            "gate_up_bytes": g1_bytes, "gate_up_flops": 2.0 * P * w.H * 2 * w.I}


def graph_time(fn, reps: int, torch, sleep_ms: float = 20.0) -> float:
    """ms per replay of fn() captured into one HIP graph (after a warm-up call
    on a side stream), replayed `reps` times back to back behind a bounded GPU
    sleep."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    g.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(sleep_ms * 2.4e6))
    t0.record()
    for _ in range(reps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    del g
    return t0.elapsed_time(t1) / reps


def step_stats(durations_ms):
    """Median, 10th and 90th percentile of per-step durations (ms)."""
    d = np.asarray(durations_ms, dtype=np.float64)
    return {"median": round(float(np.median(d)), 5), "p10": round(float(np.percentile(d, 10)), 5),
            "p90": round(float(np.percentile(d, 90)), 5), "n": int(d.size)}


def timed_steps(step, steps, torch, sleep_ms):
    """Run step(i) for i < steps back to back behind a bounded GPU sleep (so
    the host's enqueueing stays ahead of the GPU), with torch events on the
    current stream (the one the library launches on) at every step boundary.
    Returns (total ms, per-step ms list, host enqueue seconds)."""
    bounds = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda._sleep(int(sleep_ms * 2.4e6))
    h0 = time.perf_counter()
    bounds[0].record()
    for i in range(steps):
        step(i)
        bounds[i + 1].record()
    host_s = time.perf_counter() - h0
    torch.cuda.synchronize()
    per = [bounds[i].elapsed_time(bounds[i + 1]) for i in range(steps)]
    return bounds[0].elapsed_time(bounds[steps]), per, host_s


def run_workload(name: str, steps: int, warmup: int, rot: int, torch, B, S, SD, ev: HipEvents,
                 sleep_ms: float = 20.0, sample_every: int = 4) -> dict:
    w = S.WORKLOADS[name]
    T = w.T
    layers = [SD.load_layer(w, layer=l) for l in range(rot)]
    xs = [SD.activations(w, layer=l) for l in range(rot)]
    cfg = SD.config(w)
    ws = SD.workspace(cfg)
    out = torch.empty((T, w.H), dtype=torch.float32, device="cuda")
    ids = [torch.empty((T, w.top_k), dtype=torch.int32, device="cuda") for _ in range(rot)]
    wts = torch.empty((T, w.top_k), dtype=torch.float32, device="cuda")
    nst = len(B.STAGES)
    gu = B.STAGES.index("gate_up")

    def step(i, evs=None):
        r = i % rot
        L = layers[r]
        if evs is None:
            B.moe_forward(cfg, xs[r], L["router_w"], L["bias"], L["w13"], L["w13s"], L["w2"], L["w2s"], out,
                          ids[r], wts, ws)
        else:
            B.moe_forward_taps(cfg, xs[r], L["router_w"], L["bias"], L["w13"], L["w13s"], L["w2"], L["w2s"], out,
                               ids[r], wts, {"events": evs}, ws)

    # eager warmup (also runs the library's one-time kernel attribute setup)
    for i in range(max(warmup, rot)):
        step(i)
    torch.cuda.synchronize()

    # Timed region. Every `sample_every`-th step records HIP events on the
    # library's stream around its gate/up kernel (the dominant kernel); an
    # event record costs GPU time, so sampling keeps that cost out of most steps.
    g_events = []
    for i in range(steps):
        arr = (C.c_void_p * (2 * nst))()
        if i % sample_every == 0:
            pair = ev.create(2)
            arr[2 * gu], arr[2 * gu + 1] = pair[0], pair[1]
        g_events.append(arr)
    total_ms, per_step, host_s = timed_steps(lambda i: step(i, g_events[i]), steps, torch, sleep_ms)
    sampled = [i for i in range(steps) if i % sample_every == 0]
    g1_all = [ev.elapsed_ms(g_events[i][2 * gu], g_events[i][2 * gu + 1]) for i in sampled]
    g1_ms = float(np.mean(g1_all))
    for i in sampled:
        ev.destroy([g_events[i][2 * gu], g_events[i][2 * gu + 1]])

    # diagnostic breakdown (not timed): every stage bracketed by events
    d_events = [ev.create(2 * nst) for _ in range(rot)]
    torch.cuda._sleep(int(sleep_ms * 2.4e6))
    for i in range(rot):
        step(i, d_events[i])
    torch.cuda.synchronize()
    stage_ms = {s: float(np.mean([ev.elapsed_ms(d_events[i][2 * k], d_events[i][2 * k + 1]) for i in range(rot)]))
                for k, s in enumerate(B.STAGES)}
    for e in d_events:
        ev.destroy(e)

    # the same steps from a HIP graph: one graph holds the `rot` layer calls of
    # one rotation, replayed steps / rot times
    def rotation():
        for i in range(rot):
            step(i)
    graph_ms = graph_time(rotation, max(1, steps // rot), torch, sleep_ms) / rot

    # routing statistics of each rotated batch (its distinct experts set the bytes)
    distinct = []
    max_load = []
    for r in range(rot):
        a = ids[r].cpu().numpy()
        distinct.append(len(np.unique(a)))
        max_load.append(int(np.bincount(a.ravel(), minlength=w.E).max()))
    d_avg = float(np.mean([distinct[i % rot] for i in range(steps)]))
    d_sampled = float(np.mean([distinct[i % rot] for i in sampled]))
    acc = layer_accounting(w, T, d_avg, d_sampled, w.x_dtype == S.X_BF16, w.act_mode == S.ACT_INT8)
    layer_bytes, layer_flops = acc["layer_bytes"], acc["layer_flops"]
    g1_bytes, g1_flops = acc["gate_up_bytes"], acc["gate_up_flops"]
    ms_step = total_ms / steps
    return {
        "workload": name, "T": T, "steps": steps, "rot": rot, "host_enqueue_ms": host_s * 1e3,
        "gpu_bound": host_s < sleep_ms / 1e3, "gate_up_ms_min": float(np.min(g1_all)),
        "gate_up_samples": len(g1_all), "step_ms": step_stats(per_step),
        "ms_per_step": ms_step, "tokens_per_s": T / (ms_step / 1e3),
        "graph_ms_per_step": graph_ms, "graph_tokens_per_s": T / (graph_ms / 1e3),
        "stage_ms": stage_ms, "distinct_experts": d_avg, "max_load": max_load,
        "layer_alg_bytes": layer_bytes, "layer_hbm_gbs": layer_bytes / (ms_step / 1e3) / 1e9,
        "layer_fp4_tflops": layer_flops / (ms_step / 1e3) / 1e12,
        "gate_up_alg_bytes": g1_bytes, "gate_up_alg_flops": g1_flops, "gate_up_ms": g1_ms,
        "gate_up_gbs": g1_bytes / (g1_ms / 1e3) / 1e9,
        "gate_up_tflops": g1_flops / (g1_ms / 1e3) / 1e12,
    }


def run_stack(name: str, steps: int, warmup: int, torch, B, S, SD, ev: HipEvents, sleep_ms: float = 20.0,
              sample_stride: int = 4) -> dict:
    """The layer stack (x <- x + moe_l(rmsnorm(x)) over all layers, distinct
    weights per layer, all resident) through moe_forward_stack_taps. A step
    is one pass over every layer for one decode batch, starting from the same
    input stream (a 512 KB device copy at the step's start). In step i the
    layers l with l % sample_stride == i % sample_stride record HIP events on
    the library's stream around their gate/up kernel."""
    w = S.WORKLOADS[name]
    L, T = w.layers, w.T
    layers = [SD.load_layer(w, layer=l) for l in range(L)]
    cfg = SD.config(w)
    ws = torch.empty(B.moe_stack_workspace_size(cfg), dtype=torch.uint8, device="cuda")
    x0 = torch.from_numpy(S.activations(w)).cuda()
    x = x0.clone()
    nst = len(B.STAGES)
    gu = B.STAGES.index("gate_up")
    for _ in range(warmup):
        x.copy_(x0)
        B.moe_forward_stack(cfg, x, layers, ws)
    torch.cuda.synchronize()

    taps, sampled = [], []
    for i in range(steps):
        t = [None] * L
        for l in range(i % sample_stride, L, sample_stride):
            arr = (C.c_void_p * (2 * nst))()
            pair = ev.create(2)
            arr[2 * gu], arr[2 * gu + 1] = pair[0], pair[1]
            t[l] = {"events": arr}
            sampled.append((i, l, arr))
        taps.append(t)

    def step(i):
        x.copy_(x0)
        B.moe_forward_stack_taps(cfg, x, layers, ws, taps[i])
    total_ms, per_step, host_s = timed_steps(step, steps, torch, sleep_ms)
    ms_step = total_ms / steps
    g1 = [(l, ev.elapsed_ms(arr[2 * gu], arr[2 * gu + 1])) for _, l, arr in sampled]
    for _, _, arr in sampled:
        ev.destroy([arr[2 * gu], arr[2 * gu + 1]])

    # the same step replayed from one HIP graph
    def gstep():
        x.copy_(x0)
        B.moe_forward_stack(cfg, x, layers, ws)
    graph_ms = graph_time(gstep, steps, torch, sleep_ms)

    # routing of every layer of the step (diagnostic, untimed): the distinct
    # experts each layer reads set the algorithmic bytes
    x.copy_(x0)
    y = torch.empty((L, T, w.H), dtype=torch.float32, device="cuda")
    B.moe_forward_stack(cfg, x, layers, ws, layer_out=y)
    xl = x0.clone()
    rws = SD.workspace(cfg)
    xn = torch.empty_like(xl)
    ids = torch.empty((T, w.top_k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, w.top_k), dtype=torch.float32, device="cuda")
    distinct = []
    for l in range(L):
        B.moe_rmsnorm(T, w.H, xl, xn)
        B.moe_route(cfg, xn, layers[l]["router_w"], layers[l]["bias"], ids, wts, rws)
        distinct.append(len(np.unique(ids.cpu().numpy())))
        xl += y[l]
    b13, b2 = per_expert_bytes(w)
    P = T * w.top_k
    step_bytes = sum(d * (b13 + b2) + w.E * w.H * 4 + 2 * T * w.H * 4 for d in distinct)
    # gate/up launches: the layer's routed experts' W13 + int8 x as FP8 hi/lo planes + fp32 activation out
    g1_bytes = [distinct[l] * b13 + T * 2 * w.H + P * w.I * 4 for l, _ in g1]
    g1_ms = [d for _, d in g1]
    del layers
    return {"workload": name, "layers": L, "T": T, "steps": steps, "ms_per_step": ms_step,
            "step_ms": step_stats(per_step), "tokens_per_s": T / (ms_step / 1e3), "host_enqueue_ms": host_s * 1e3,
            "graph_ms_per_step": graph_ms, "graph_tokens_per_s": T / (graph_ms / 1e3),
            "gpu_bound": host_s * 1e3 < sleep_ms + total_ms,
            "distinct_experts_per_layer": float(np.mean(distinct)), "step_alg_bytes": step_bytes,
            "hbm_gbs": step_bytes / (ms_step / 1e3) / 1e9, "graph_hbm_gbs": step_bytes / (graph_ms / 1e3) / 1e9,
            "gate_up_launches": len(g1), "gate_up_ms": float(np.mean(g1_ms)),
            "gate_up_alg_bytes": float(np.mean(g1_bytes)),
            "gate_up_gbs": float(np.sum(g1_bytes)) / (float(np.sum(g1_ms)) / 1e3) / 1e9}


def run_ep_rank(name: str, ranks: int, steps: int, warmup: int, torch, B, S, SD, sleep_ms: float = 20.0) -> dict:
    """One rank's share under expert parallelism over `ranks` GPUs: the batch
    is routed over all experts (the router replicated), experts are placed in
    contiguous blocks of E/ranks, and the heaviest rank computes the pairs
    routed to its block -- one row per pair, top_k = 1, its slice of the
    weights -- through moe_forward_routed. The dispatch and return exchanges
    are not part of it. A step is one such call."""
    w = S.WORKLOADS[name]
    lay = SD.load_layer(w)
    cfg = SD.config(w)
    x = SD.activations(w)
    ids = torch.empty((w.T, w.top_k), dtype=torch.int32, device="cuda")
    wts = torch.empty((w.T, w.top_k), dtype=torch.float32, device="cuda")
    B.moe_route(cfg, x, lay["router_w"], lay["bias"], ids, wts, SD.workspace(cfg))
    ids_h, w_h = ids.cpu().numpy().ravel(), wts.cpu().numpy().ravel()
    per = w.E // ranks
    load = np.bincount(ids_h // per, minlength=ranks)
    r = int(np.argmax(load))
    pairs = np.nonzero(ids_h // per == r)[0]
    tok = torch.from_numpy(pairs // w.top_k).cuda()
    x_rows = x[tok].contiguous()
    ids_l = torch.from_numpy((ids_h[pairs] - per * r).astype(np.int32).reshape(-1, 1)).cuda()
    w_l = torch.from_numpy(w_h[pairs].astype(np.float32).reshape(-1, 1)).cuda()
    local = {n: lay[n].view(w.E, -1)[per * r:per * (r + 1)].contiguous() for n in ("w13", "w13s", "w2", "w2s")}
    del lay
    Pl = len(pairs)
    lcfg = B.make_config(Pl, w.H, w.I, per, 1, w.x_dtype, w.act_mode, B.MOE_LAYOUT_PREPACKED)
    ws = SD.workspace(lcfg)
    out = torch.empty((Pl, w.H), dtype=torch.float32, device="cuda")

    def step():
        B.moe_forward_routed(lcfg, x_rows, ids_l, w_l, local["w13"], local["w13s"], local["w2"], local["w2s"], out,
                             ws)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(sleep_ms * 2.4e6))
    t0.record()
    for _ in range(steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    b13, b2 = per_expert_bytes(w)
    flops = 2.0 * Pl * (w.H * 2 * w.I + w.I * w.H)
    used = len(np.unique(ids_h[pairs]))
    return {"workload": f"{name} on rank {r} of {ranks} (experts {per * r}..{per * (r + 1) - 1})", "pairs": Pl,
            "pair_share": Pl / len(ids_h), "experts_used": used, "ms_per_step": ms,
            "pairs_per_s": Pl / (ms / 1e3), "fp4_tflops": flops / (ms / 1e3) / 1e12,
            "hbm_gbs": used * (b13 + b2) / (ms / 1e3) / 1e9}


def run_dense(name: str, steps: int, warmup: int, torch, B, S, sleep_ms: float = 20.0) -> dict:
    """The block-scaled FP8 dense projection on prepacked weights: a step is
    one moe_dense_fp8_forward (quantize x, then the GEMM); the GEMM alone is
    timed by events around moe_dense_fp8_gemm on pre-quantized rows (for
    M > 32 that call is the wide kernel alone)."""
    w = S.DENSE_WORKLOADS[name]
    wq_h, ws_h = S.dense_weights(w)
    wq, ws = torch.from_numpy(wq_h).cuda(), torch.from_numpy(ws_h).cuda()
    cb, sb = B.moe_dense_fp8_prepacked_size(w.N, w.K)
    pw = torch.empty(cb, dtype=torch.uint8, device="cuda")
    ps = torch.empty(sb, dtype=torch.uint8, device="cuda")
    B.moe_dense_fp8_prepack(w.N, w.K, wq, ws, pw, ps)
    del wq, ws
    x = torch.from_numpy(S.dense_activations(w)).cuda()
    cfg = B.make_dense_config(w.M, w.N, w.K, w.x_dtype, B.MOE_LAYOUT_PREPACKED)
    work = torch.empty(B.moe_dense_fp8_workspace_size(cfg), dtype=torch.uint8, device="cuda")
    y = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
    xq = torch.empty((w.M, w.K), dtype=torch.uint8, device="cuda")
    xs = torch.empty((w.M, w.K // 32), dtype=torch.uint8, device="cuda")
    B.moe_dense_fp8_quantize(w.M, w.K, w.x_dtype, x, xq, xs)
    for _ in range(warmup):
        B.moe_dense_fp8_forward(cfg, x, pw, ps, y, work)
    torch.cuda.synchronize()
    total_ms, per, _ = timed_steps(lambda i: B.moe_dense_fp8_forward(cfg, x, pw, ps, y, work), steps, torch, sleep_ms)
    _, per_gemm, _ = timed_steps(lambda i: B.moe_dense_fp8_gemm(cfg, xq, xs, pw, ps, y, work), steps, torch, sleep_ms)
    fwd_ms, gemm_ms = total_ms / steps, float(np.mean(per_gemm))
    flops = 2.0 * w.M * w.N * w.K
    wbytes = w.N * w.K * (1 + 1 / 32)
    xbytes = w.M * w.K * (2 if w.x_dtype == S.X_BF16 else 4)
    gemm_bytes = wbytes + w.M * w.K * (1 + 1 / 32) + w.M * w.N * 4
    return {"workload": name, "M": w.M, "N": w.N, "K": w.K, "steps": steps,
            "ms_per_step": fwd_ms, "step_ms": step_stats(per), "tokens_per_s": w.M / (fwd_ms / 1e3),
            "fwd_tflops": flops / (fwd_ms / 1e3) / 1e12,
            "fwd_hbm_gbs": (wbytes + xbytes + w.M * w.N * 4) / (fwd_ms / 1e3) / 1e9,
            "gemm_ms": gemm_ms, "gemm_step_ms": step_stats(per_gemm), "gemm_alg_flops": flops,
            "gemm_alg_bytes": gemm_bytes, "gemm_tflops": flops / (gemm_ms / 1e3) / 1e12,
            "gemm_gbs": gemm_bytes / (gemm_ms / 1e3) / 1e9}


def dense_summary(v: dict) -> dict:
    return {"M": v["M"], "N": v["N"], "K": v["K"], "tokens_per_s": round(v["tokens_per_s"], 1),
            "ms_per_step": round(v["ms_per_step"], 5), "step_ms": v["step_ms"],
            "fwd_fp8_tflops": round(v["fwd_tflops"], 1), "fwd_fp8_frac": round(v["fwd_tflops"] / FP8_PEAK_TFLOPS, 4),
            "fwd_hbm_gbs": round(v["fwd_hbm_gbs"], 1), "fwd_hbm_frac": round(v["fwd_hbm_gbs"] / HBM_PEAK_GBS, 4),
            "gemm_us": round(v["gemm_ms"] * 1e3, 2), "gemm_fp8_tflops": round(v["gemm_tflops"], 1),
            "gemm_fp8_frac": round(v["gemm_tflops"] / FP8_PEAK_TFLOPS, 4), "gemm_gbs": round(v["gemm_gbs"], 1)}


def cpu_baseline(name: str, budget_s: float, S, oracle) -> dict:
    """The oracle, untuned, on the host cores, on a bounded sample of the
    same workload: for the layer stack, consecutive layers of the stack on
    the same 32-token stream (rmsnorm, the layer, the residual add, each
    layer's expert weights generated outside the timed region) scaled to
    whole-stack steps; for a single layer, whole-layer calls on (at most 64 of)
    its tokens (every output depends only on its own token)."""
    w = S.WORKLOADS[name]
    if w.layers > 1:
        from concurrent.futures import ThreadPoolExecutor
        x = S.activations(w)
        t_layers, l = 0.0, 0
        while l < w.layers and (l == 0 or t_layers < budget_s):
            wr, b = S.router_weights(w, l), S.router_bias(w, l)
            ids, _ = oracle.route(oracle.rmsnorm(x), wr, b, w.top_k)  # only to know which experts to generate
            need = sorted(set(np.unique(ids).tolist()))
            with ThreadPoolExecutor(16) as ex:
                got = dict(zip(need, ex.map(lambda e: S.expert_weights(w, l, e), need)))
            ex_w = [got.get(e) for e in range(w.E)]
            t0 = time.perf_counter()
            xn = oracle.rmsnorm(x)
            y = oracle.moe_layer(xn, wr, b, ex_w, w.top_k, w.act_mode)["out"]
            x = (x + y).astype(np.float32)
            t_layers += time.perf_counter() - t0
            l += 1
        per_step = t_layers / l * w.layers
        return {"value": w.T / per_step, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
                "sample": f"layers 0..{l - 1} of the {w.layers}-layer stack on its {w.T}-token stream "
                          f"(rmsnorm + layer + residual), {t_layers:.1f} s of oracle work, scaled to "
                          f"{w.layers}-layer steps; expert weight generation outside the timed region"}
    T = min(w.T, 64)
    batches = []
    for l in range(4):
        x = S.activations(w, l, T=w.T)[:T]
        wr, b = S.router_weights(w, l), S.router_bias(w, l)
        ids, _ = oracle.route(x, wr, b, w.top_k)
        need = set(np.unique(ids).tolist())
        ex = [S.expert_weights(w, l, e) if e in need else None for e in range(w.E)]
        batches.append((x, wr, b, ex))
    n_tok = 0
    t0 = time.perf_counter()
    i = 0
    while True:
        x, wr, b, ex = batches[i % len(batches)]
        oracle.moe_layer(x, wr, b, ex, w.top_k, w.act_mode)
        n_tok += x.shape[0]
        i += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": n_tok / el, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{i} whole-layer oracle calls of {name} ({T} tokens each, 4 seeded batches rotating), "
                      f"{el:.1f} s wall, weight generation outside the timed region"}


def profiled(kernel: str, workload: str):
    """The committed rocprofv3 counter record of a kernel on a workload (HBM
    bytes per launch, MFMA utilisation), if the kernel's source is unchanged
    since the counters were taken."""
    if not os.path.exists(PROFILE_TRAFFIC):
        return None
    try:
        rec = json.load(open(PROFILE_TRAFFIC))[f"{kernel}@{workload}"]
    except (KeyError, ValueError):
        return None
    import hashlib
    src = os.path.join(ROOT, "fp4_routed_mixture_amd", "csrc", rec["source"])
    if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != rec["source_sha256"]:
        return None
    return rec


def streaming_read_gbs(torch, SD, gib: int = 8, reps: int = 5) -> float:
    """A plain streaming read of a large buffer (nontemporal 16-byte loads,
    8 workgroups of 256 threads per CU): the practical HBM read ceiling
    beside the 8 TB/s peak."""
    buf = torch.empty(gib << 30, dtype=torch.uint8, device="cuda")
    blocks = 256 * 8
    sink = torch.empty(blocks * 16, dtype=torch.uint8, device="cuda")
    SD.stream_read(buf, blocks, sink)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        SD.stream_read(buf, blocks, sink)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps
    del buf, sink
    return (gib << 30) / (ms / 1e3) / 1e9


def mfma_probe(torch, SD, iters: int = 40000) -> dict:
    """MFMA issue rate on random operands -- the scaled 32x32x64 on FP4 and
    FP8, the 32x32x2 on fp32 (the router's) -- with one and two waves per
    SIMD: TFLOP/s from events and the shader clock measured in-kernel
    (s_memtime cycles over the 100 MHz s_memrealtime)."""
    res = {}
    for fmt, n, flop in (("fp4", iters, 131072.0), ("fp8", iters // 2, 131072.0), ("fp32", iters // 4, 4096.0)):
        for per_simd in (1, 2):
            blocks = 256 * per_simd  # 4 waves a workgroup: one per SIMD
            out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
            clocks = torch.empty(blocks * 8, dtype=torch.int64, device="cuda")
            SD.mfma_probe(blocks, 100, out, clocks, fmt)
            torch.cuda.synchronize()
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record()
            SD.mfma_probe(blocks, n, out, clocks, fmt)
            t1.record()
            torch.cuda.synchronize()
            ms = t0.elapsed_time(t1)
            flops = blocks * 4 * n * 8 * flop
            c = clocks.view(-1, 2).cpu().numpy().astype(np.float64)
            mhz = c[:, 0] / (c[:, 1] / 100.0)
            key = f"waves_per_simd_{per_simd}" if fmt == "fp4" else f"{fmt}_waves_per_simd_{per_simd}"
            res[key] = {
                "tflops": round(flops / (ms / 1e3) / 1e12, 1), "ms": round(ms, 3),
                "shader_mhz_median": round(float(np.median(mhz)), 1),
                "cycles_per_mfma_per_simd": round(float(np.median(c[:, 0])) / (n * 8 * per_simd), 2)}
    return res


def leg_summary(v: dict) -> dict:
    return {"tokens_per_s": round(v["tokens_per_s"], 1), "ms_per_step": round(v["ms_per_step"], 5),
            "step_ms": v["step_ms"],
            "graph_tokens_per_s": round(v["graph_tokens_per_s"], 1),
            "graph_ms_per_step": round(v["graph_ms_per_step"], 5),
            "layer_hbm_gbs": round(v["layer_hbm_gbs"], 1),
            "layer_hbm_frac": round(v["layer_hbm_gbs"] / HBM_PEAK_GBS, 4),
            "layer_fp4_tflops": round(v["layer_fp4_tflops"], 1),
            "layer_fp4_frac": round(v["layer_fp4_tflops"] / FP4_PEAK_TFLOPS, 4),
            "gate_up_gbs": round(v["gate_up_gbs"], 1), "gate_up_tflops": round(v["gate_up_tflops"], 1),
            "stage_us": {s: round(x * 1e3, 2) for s, x in v["stage_ms"].items()},
            "distinct_experts": v["distinct_experts"]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="stack43_decode_t32",
                    help="headline workload: the 43-layer decode stack (default) or a single-layer workload")
    ap.add_argument("--rot", type=int, default=8, help="distinct layers cycled through (single-layer workloads)")
    ap.add_argument("--legs", default="prefill_t16384_zipf,decode_t4,decode_t64_zipf,prefill_t4604_zipf,"
                                      "decode_t4_tp4,prefill_t4604_zipf_tp4,prefill_t4604_zipf_ep8,"
                                      "dense_t16384,dense_t4604,dense_t32",
                    help="comma-separated legs to run after the headline workload ('' for none)")
    ap.add_argument("--no-legs", action="store_true", help="run the headline workload only")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--mfma-probe", action="store_true",
                    help="only run the FP4 MFMA rate / shader clock probe and print its JSON")
    ap.add_argument("--dense", default="",
                    help="only run the named dense FP8 projection workload (--steps, --warmup) and print its JSON")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy three times (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the layer is not sharded here",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X (no HIP device visible)", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel(), "launches": 3}))
        return
    from fp4_routed_mixture_amd import binding as B
    from fp4_routed_mixture_amd import synth as S
    from fp4_routed_mixture_amd import synth_device as SD
    if args.mfma_probe:
        print(json.dumps(mfma_probe(torch, SD)))
        return
    if args.dense:
        print(json.dumps(dense_summary(run_dense(args.dense, args.steps, args.warmup, torch, B, S))))
        return
    B.lib()
    ev = HipEvents()
    w = S.WORKLOADS[args.workload]
    stack_head = w.layers > 1

    if stack_head:
        head = run_stack(args.workload, args.steps, args.warmup, torch, B, S, SD, ev)
        print(f"# {args.workload}: {head['ms_per_step']:.3f} ms/step ({w.layers} layers), "
              f"{head['tokens_per_s']:.0f} tok/s, {head['hbm_gbs']:.0f} GB/s; graph {head['graph_ms_per_step']:.3f} "
              f"ms/step; gate/up {head['gate_up_gbs']:.0f} GB/s", file=sys.stderr, flush=True)
    else:
        head = run_workload(args.workload, args.steps, args.warmup, args.rot, torch, B, S, SD, ev)
        print(f"# {args.workload}: {head['ms_per_step'] * 1e3:.1f} us/step, {head['tokens_per_s']:.0f} tok/s",
              file=sys.stderr, flush=True)
    torch.cuda.empty_cache()
    legs = {}
    want = set() if args.no_legs else set(x for x in args.legs.split(",") if x)
    for name, steps, rot in (("prefill_t16384_zipf", 8, 2), ("decode_t4", 64, 8), ("decode_t64_zipf", 32, 8),
                             ("prefill_t4604_zipf", 10, 2), ("decode_t4_tp4", 64, 8),
                             ("prefill_t4604_zipf_tp4", 10, 2)):
        if name not in want or name == args.workload:
            continue
        torch.cuda.empty_cache()
        r = run_workload(name, steps, 3, rot, torch, B, S, SD, ev, sample_every=1 if "prefill" in name else 4)
        legs[name] = r
        print(f"# {name}: {r['ms_per_step'] * 1e3:.1f} us/step (graph {r['graph_ms_per_step'] * 1e3:.1f}), "
              f"{r['tokens_per_s']:.0f} tok/s, layer {r['layer_hbm_gbs']:.0f} GB/s, {r['layer_fp4_tflops']:.0f} TF/s; "
              f"stages(us) " + " ".join(f"{k}={v * 1e3:.1f}" for k, v in r["stage_ms"].items()),
              file=sys.stderr, flush=True)
    ep = None
    if "prefill_t4604_zipf_ep8" in want:
        torch.cuda.empty_cache()
        ep = run_ep_rank("prefill_t4604_zipf", 8, 10, 2, torch, B, S, SD)
        print(f"# prefill_t4604_zipf_ep8: {ep['ms_per_step'] * 1e3:.1f} us/step, {ep['pairs']} pairs "
              f"({100 * ep['pair_share']:.1f}% of all), {ep['fp4_tflops']:.0f} TF/s", file=sys.stderr, flush=True)
    dense = {}
    for name, steps in (("dense_t16384", 20), ("dense_t4604", 20), ("dense_t32", 50)):
        if name not in want:
            continue
        torch.cuda.empty_cache()
        d = run_dense(name, steps, 3, torch, B, S)
        dense[name] = d
        print(f"# {name}: forward {d['ms_per_step'] * 1e3:.1f} us ({d['fwd_tflops']:.0f} TF/s, "
              f"{d['fwd_hbm_gbs']:.0f} GB/s), GEMM {d['gemm_ms'] * 1e3:.1f} us ({d['gemm_tflops']:.0f} TF/s)",
              file=sys.stderr, flush=True)
    torch.cuda.empty_cache()
    stream_gbs = streaming_read_gbs(torch, SD)

    # roofline of the dominant kernel of the headline workload
    if stack_head:
        kernel = "decode_gate_up_kernel"
        prof = profiled(kernel, args.workload)
        roof = {"bound": "hbm", "kernel": kernel, "achieved": round(head["gate_up_gbs"], 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(head["gate_up_gbs"] / HBM_PEAK_GBS, 4),
                "traffic": prof["bytes_per_launch"] if prof else None,
                "alg_bytes_per_launch": round(head["gate_up_alg_bytes"]), "launches_timed": head["gate_up_launches"],
                "avg_launch_us": round(head["gate_up_ms"] * 1e3, 2),
                "step_hbm_gbs": round(head["hbm_gbs"], 1), "step_hbm_frac": round(head["hbm_gbs"] / HBM_PEAK_GBS, 4),
                "streaming_read_gbs": round(stream_gbs, 1)}
    else:
        mx = w.act_mode == S.ACT_MXFP4
        kernel = "prefill_gemm_kernel<true>" if mx else "decode_gate_up_kernel"
        prof = profiled(kernel, args.workload)
        ach, peak, unit, bound = ((head["gate_up_tflops"], FP4_PEAK_TFLOPS, "TFLOP/s", "mfma") if mx else
                                  (head["gate_up_gbs"], HBM_PEAK_GBS, "GB/s", "hbm"))
        roof = {"bound": bound, "kernel": kernel, "achieved": round(ach, 1), "peak": peak, "unit": unit,
                "frac": round(ach / peak, 4), "traffic": prof["bytes_per_launch"] if prof else None,
                "avg_launch_us": round(head["gate_up_ms"] * 1e3, 2),
                "layer_hbm_frac": round(head["layer_hbm_gbs"] / HBM_PEAK_GBS, 4),
                "streaming_read_gbs": round(stream_gbs, 1)}
    # the prefill chunk's FP4 roofline (the metric's "prefill FP4 MFMA % of peak")
    roof_pf = None
    pf = legs.get("prefill_t16384_zipf") or (head if args.workload == "prefill_t16384_zipf" else None)
    if pf is not None:
        k = "prefill_gemm_kernel<true>"
        prof = profiled(k, "prefill_t16384_zipf")
        roof_pf = {"bound": "mfma", "kernel": k, "workload": "prefill_t16384_zipf",
                   "achieved": round(pf["gate_up_tflops"], 1), "peak": FP4_PEAK_TFLOPS, "unit": "TFLOP/s",
                   "frac": round(pf["gate_up_tflops"] / FP4_PEAK_TFLOPS, 4),
                   "traffic": prof["bytes_per_launch"] if prof else None,
                   "mfma_util_profiled": prof.get("mfma_util") if prof else None,
                   "alg_flops_per_launch": pf["gate_up_alg_flops"], "avg_launch_us": round(pf["gate_up_ms"] * 1e3, 2),
                   "launches_timed": pf["gate_up_samples"],
                   "layer_fp4_tflops": round(pf["layer_fp4_tflops"], 1),
                   "layer_fp4_frac": round(pf["layer_fp4_tflops"] / FP4_PEAK_TFLOPS, 4),
                   "layer_tokens_per_s": round(pf["tokens_per_s"], 1)}

    # the dense FP8 projection's GEMM at 16,384 tokens against the FP8 peak
    roof_dense = None
    if "dense_t16384" in dense:
        d = dense["dense_t16384"]
        k = "dense_fp8_wide_kernel<true,4>"
        prof = profiled(k, "dense_t16384")
        roof_dense = {"bound": "mfma", "kernel": k, "workload": "dense_t16384", "achieved": round(d["gemm_tflops"], 1),
                      "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(d["gemm_tflops"] / FP8_PEAK_TFLOPS, 4),
                      "traffic": prof["bytes_per_launch"] if prof else None,
                      "alg_flops_per_launch": d["gemm_alg_flops"], "avg_launch_us": round(d["gemm_ms"] * 1e3, 2),
                      "launches_timed": d["steps"]}

    import oracle
    cpu = cpu_baseline(args.workload, args.cpu_seconds, S, oracle)

    line = {
        "metric": "routed-MoE tokens/s; decode HBM GB/s and prefill FP4 MFMA % of peak",
        "value": round(head["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": head["steps"],
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "step_ms": head["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4" if w.act_mode == S.ACT_MXFP4 else "fp4xint8",
        "data": "synthetic",
        "config": {"workload": args.workload, "layers": w.layers, "T": w.T, "H": w.H, "I": w.I, "E": w.E,
                   "top_k": w.top_k, "x": "bf16" if w.x_dtype == S.X_BF16 else "fp32",
                   "act": "mxfp4" if w.act_mode == S.ACT_MXFP4 else "int8",
                   "routing": "zipf1.1" if w.zipf else "uniform"},
        "roofline": roof,
        "roofline_prefill": roof_pf,
        "roofline_dense": roof_dense,
        "cpu_baseline": cpu,
        "graph": {"ms_per_step": round(head["graph_ms_per_step"], 5),
                  "tokens_per_s": round(head["graph_tokens_per_s"], 1)},
        "legs": {k: leg_summary(v) for k, v in legs.items()},
    }
    for k, v in dense.items():
        line["legs"][k] = dense_summary(v)
    if not stack_head:
        line["stage_us_diagnostic"] = {k: round(v * 1e3, 2) for k, v in head["stage_ms"].items()}
    else:
        line["distinct_experts_per_layer"] = head["distinct_experts_per_layer"]
    if ep is not None:
        line["legs"]["prefill_t4604_zipf_ep8"] = {
            "workload": ep["workload"], "pairs": ep["pairs"], "pair_share": round(ep["pair_share"], 4),
            "experts_used": ep["experts_used"], "ms_per_step": round(ep["ms_per_step"], 5),
            "pairs_per_s": round(ep["pairs_per_s"], 1), "fp4_tflops": round(ep["fp4_tflops"], 1),
            "fp4_frac": round(ep["fp4_tflops"] / FP4_PEAK_TFLOPS, 4), "hbm_gbs": round(ep["hbm_gbs"], 1)}
    print(json.dumps(line))


if __name__ == "__main__":
    main()
