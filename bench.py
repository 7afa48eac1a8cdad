#!/usr/bin/env python
"""Benchmark of the FP4 routed-MoE layer on one MI355X.

A step is one moe_forward (route, sort, quantize, gate/up GEMM with SiLU*mul,
down GEMM, combine) over one batch. The headline workload is the decode layer
with 4 tokens (hidden 4096, intermediate 2048, 256 experts, top-6, bf16 x,
int8 activations). Steps cycle through ROT distinct layers (weights and
inputs drawn from different seeds' streams) so each step streams expert
weights that the previous steps did not touch, as a 43-layer model's decode
does; the 256 MB last-level cache cannot serve them.

Prints one JSON line: tokens/s, the dominant kernel's roofline fraction
(algorithmic bytes or FLOPs per launch / its average duration from HIP events
recorded on the library's stream inside the timed region), and the CPU
oracle's tokens/s on a bounded sample of the same workload.
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

    # Timed region: a bounded GPU sleep first keeps the device busy while the
    # host enqueues all `steps` layer calls, so the steps then run back to
    # back and the measured time is the GPU's, not the host's launch rate.
    # Every `sample_every`-th step records HIP events on the library's stream
    # around its gate/up kernel (the dominant kernel); an event record costs
    # GPU time, so sampling keeps that cost out of most steps.
    g_events = []
    for i in range(steps):
        arr = (C.c_void_p * (2 * nst))()
        if i % sample_every == 0:
            pair = ev.create(2)
            arr[2 * gu], arr[2 * gu + 1] = pair[0], pair[1]
        g_events.append(arr)
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(sleep_ms * 2.4e6))
    t_start.record()
    h0 = time.perf_counter()
    for i in range(steps):
        step(i, g_events[i])
    host_s = time.perf_counter() - h0
    t_end.record()
    torch.cuda.synchronize()
    elapsed = t_start.elapsed_time(t_end) / 1e3
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
    b13, b2 = per_expert_bytes(w)
    xbytes = T * w.H * (2 if w.x_dtype == S.X_BF16 else 4)
    P = T * w.top_k
    layer_bytes = d_avg * (b13 + b2) + w.E * w.H * 4 + xbytes + T * w.H * 4
    # gate/up kernel: weights of the routed experts + quantized x in + its output
    if w.act_mode == S.ACT_INT8:
        g1_bytes = d_avg * b13 + T * 2 * w.H + P * w.I * 4
    else:
        g1_bytes = d_avg * b13 + T * w.H // 2 + T * w.H // 32 + P * (w.I // 2 + w.I // 32)
    g1_flops = 2.0 * P * w.H * 2 * w.I
    layer_flops = 2.0 * P * (w.H * 2 * w.I + w.I * w.H)
    ms_step = elapsed * 1e3 / steps
    return {
        "workload": name, "T": T, "steps": steps, "rot": rot, "host_enqueue_ms": host_s * 1e3,
        "gpu_bound": host_s < sleep_ms / 1e3, "gate_up_ms_min": float(np.min(g1_all)),
        "gate_up_samples": len(g1_all),
        "ms_per_step": ms_step, "tokens_per_s": T / (ms_step / 1e3),
        "graph_ms_per_step": graph_ms, "graph_tokens_per_s": T / (graph_ms / 1e3),
        "stage_ms": stage_ms, "distinct_experts": d_avg, "max_load": max_load,
        "layer_alg_bytes": layer_bytes, "layer_hbm_gbs": layer_bytes / (ms_step / 1e3) / 1e9,
        "layer_fp4_tflops": layer_flops / (ms_step / 1e3) / 1e12,
        "gate_up_alg_bytes": g1_bytes, "gate_up_ms": g1_ms,
        "gate_up_gbs": g1_bytes / (g1_ms / 1e3) / 1e9,
        "gate_up_tflops": g1_flops / (g1_ms / 1e3) / 1e12,
    }


def run_stack(name: str, steps: int, warmup: int, torch, B, S, SD, sleep_ms: float = 20.0) -> dict:
    """The layer stack (x <- x + moe_l(rmsnorm(x)) over all layers, distinct
    weights per layer, all resident) through moe_forward_stack. A step is one
    pass over every layer for one decode batch."""
    w = S.WORKLOADS[name]
    L, T = w.layers, w.T
    layers = [SD.load_layer(w, layer=l) for l in range(L)]
    cfg = SD.config(w)
    ws = torch.empty(B.moe_stack_workspace_size(cfg), dtype=torch.uint8, device="cuda")
    x0 = torch.from_numpy(S.activations(w)).cuda()
    x = x0.clone()
    for _ in range(warmup):
        B.moe_forward_stack(cfg, x, layers, ws)
    torch.cuda.synchronize()
    x.copy_(x0)
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(sleep_ms * 2.4e6))
    t_start.record()
    h0 = time.perf_counter()
    for _ in range(steps):
        B.moe_forward_stack(cfg, x, layers, ws)
    host_s = time.perf_counter() - h0
    t_end.record()
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / steps
    # the same step (all layers) replayed from one HIP graph
    graph_ms = graph_time(lambda: B.moe_forward_stack(cfg, x, layers, ws), steps, torch, sleep_ms)

    # routing of every layer on the first step's stream (diagnostic, untimed):
    # the distinct experts each layer reads set the algorithmic bytes
    x.copy_(x0)
    y = torch.empty((L, T, w.H), dtype=torch.float32, device="cuda")
    B.moe_forward_stack(cfg, x, layers, ws, layer_out=y)
    xl = x0.clone()
    rcfg = SD.config(w)
    rws = SD.workspace(rcfg)
    xn = torch.empty_like(xl)
    ids = torch.empty((T, w.top_k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, w.top_k), dtype=torch.float32, device="cuda")
    distinct = []
    for l in range(L):
        B.moe_rmsnorm(T, w.H, xl, xn)
        B.moe_route(rcfg, xn, layers[l]["router_w"], layers[l]["bias"], ids, wts, rws)
        distinct.append(len(np.unique(ids.cpu().numpy())))
        xl += y[l]
    b13, b2 = per_expert_bytes(w)
    step_bytes = sum(d * (b13 + b2) + w.E * w.H * 4 + 2 * T * w.H * 4 for d in distinct)
    del layers
    return {"workload": name, "layers": L, "T": T, "steps": steps, "ms_per_step": ms_step,
            "tokens_per_s": T / (ms_step / 1e3), "host_enqueue_ms": host_s * 1e3 / steps,
            "graph_ms_per_step": graph_ms, "graph_tokens_per_s": T / (graph_ms / 1e3),
            "gpu_bound": host_s < sleep_ms / 1e3 + steps * ms_step / 1e3,
            "distinct_experts_per_layer": float(np.mean(distinct)), "step_alg_bytes": step_bytes,
            "hbm_gbs": step_bytes / (ms_step / 1e3) / 1e9, "graph_hbm_gbs": step_bytes / (graph_ms / 1e3) / 1e9}


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


def cpu_baseline(name: str, budget_s: float, S, oracle) -> dict:
    """The oracle, untuned, on the host cores: whole layers of the same
    workload (rotating the same seeded batches) until about budget_s of CPU
    work; for large batches a token sample (every output depends only on its
    own token)."""
    w = S.WORKLOADS[name]
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


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if the
    kernel source is unchanged since they were taken."""
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
    return rec["bytes_per_launch"]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_t4")
    ap.add_argument("--rot", type=int, default=8, help="distinct layers cycled through")
    ap.add_argument("--no-legs", action="store_true", help="skip the prefill and Zipf-decode legs")
    ap.add_argument("--legs", default="decode_t64_zipf,prefill_t4604_zipf,prefill_t16384_zipf,stack43_decode_t32,"
                                      "decode_t4_tp4,prefill_t4604_zipf_tp4,prefill_t4604_zipf_ep8",
                    help="comma-separated legs to run after the headline workload")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
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
    B.lib()
    ev = HipEvents()

    main_res = run_workload(args.workload, args.steps, args.warmup, args.rot, torch, B, S, SD, ev)
    print(f"# {args.workload}: {main_res['ms_per_step'] * 1e3:.1f} us/step, {main_res['tokens_per_s']:.0f} tok/s "
          f"(graph {main_res['graph_ms_per_step'] * 1e3:.1f} us/step), stages(us) " + " ".join(f"{k}={v * 1e3:.1f}" for k, v in main_res["stage_ms"].items()),
          file=sys.stderr, flush=True)
    legs = {}
    want = set() if args.no_legs else set(args.legs.split(","))
    stack = None
    if want:
        for name, steps, rot in (("decode_t64_zipf", 32, 8), ("prefill_t4604_zipf", 10, 2),
                                 ("prefill_t16384_zipf", 4, 2), ("decode_t4_tp4", 64, 8),
                                 ("prefill_t4604_zipf_tp4", 10, 2)):
            if name not in want:
                continue
            torch.cuda.empty_cache()
            r = run_workload(name, steps, 3, rot, torch, B, S, SD, ev)
            legs[name] = r
            print(f"# {name}: {r['ms_per_step'] * 1e3:.1f} us/step (graph {r['graph_ms_per_step'] * 1e3:.1f}), "
                  f"{r['tokens_per_s']:.0f} tok/s, layer {r['layer_hbm_gbs']:.0f} GB/s, {r['layer_fp4_tflops']:.0f} TF/s; stages(us) "
                  + " ".join(f"{k}={v * 1e3:.1f}" for k, v in r["stage_ms"].items()), file=sys.stderr, flush=True)
    ep = None
    if "prefill_t4604_zipf_ep8" in want:
        torch.cuda.empty_cache()
        ep = run_ep_rank("prefill_t4604_zipf", 8, 10, 2, torch, B, S, SD)
        print(f"# prefill_t4604_zipf_ep8: {ep['ms_per_step'] * 1e3:.1f} us/step, {ep['pairs']} pairs "
              f"({100 * ep['pair_share']:.1f}% of all), {ep['fp4_tflops']:.0f} TF/s, {ep['hbm_gbs']:.0f} GB/s",
              file=sys.stderr, flush=True)
    if "stack43_decode_t32" in want:
        torch.cuda.empty_cache()
        stack = run_stack("stack43_decode_t32", 5, 1, torch, B, S, SD)
        print(f"# stack43_decode_t32: {stack['ms_per_step']:.2f} ms/step (43 layers), {stack['tokens_per_s']:.0f} "
              f"tok/s, {stack['hbm_gbs']:.0f} GB/s; graph {stack['graph_ms_per_step']:.2f} ms/step, "
              f"{stack['graph_tokens_per_s']:.0f} tok/s", file=sys.stderr, flush=True)

    w = S.WORKLOADS[args.workload]
    mx = w.act_mode == S.ACT_MXFP4
    if mx:
        ach, peak, unit, bound = main_res["gate_up_tflops"], FP4_PEAK_TFLOPS, "TFLOP/s", "mfma"
    else:
        ach, peak, unit, bound = main_res["gate_up_gbs"], HBM_PEAK_GBS, "GB/s", "hbm"
    kernel = "prefill_gemm_kernel<true>" if mx else "decode_gate_up_kernel"
    roof = {"bound": bound, "kernel": kernel, "achieved": round(ach, 1), "peak": peak, "unit": unit,
            "frac": round(ach / peak, 4), "traffic": traffic_for(kernel, args.workload),
            "layer_hbm_gbs": round(main_res["layer_hbm_gbs"], 1),
            "layer_hbm_frac": round(main_res["layer_hbm_gbs"] / HBM_PEAK_GBS, 4)}

    import oracle
    cpu = cpu_baseline(args.workload, args.cpu_seconds, S, oracle)

    line = {
        "metric": "routed-MoE tokens/s; decode HBM GB/s and prefill FP4 MFMA % of peak",
        "value": round(main_res["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": main_res["steps"],
        "warmup": args.warmup,
        "ms_per_step": round(main_res["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4" if mx else "fp4xint8",
        "data": "synthetic",
        "config": {"workload": args.workload, "T": w.T, "H": w.H, "I": w.I, "E": w.E, "top_k": w.top_k,
                   "x": "bf16" if w.x_dtype == S.X_BF16 else "fp32", "act": "mxfp4" if mx else "int8",
                   "routing": "zipf1.1" if w.zipf else "uniform", "distinct_layers_cycled": args.rot},
        "roofline": roof,
        "cpu_baseline": cpu,
        "graph": {"ms_per_step": round(main_res["graph_ms_per_step"], 5),
                  "tokens_per_s": round(main_res["graph_tokens_per_s"], 1)},
        "stage_us_diagnostic": {k: round(v * 1e3, 2) for k, v in main_res["stage_ms"].items()},
        "distinct_experts": main_res["distinct_experts"],
        "legs": {k: {"tokens_per_s": round(v["tokens_per_s"], 1), "ms_per_step": round(v["ms_per_step"], 5),
                     "graph_tokens_per_s": round(v["graph_tokens_per_s"], 1),
                     "graph_ms_per_step": round(v["graph_ms_per_step"], 5),
                     "layer_hbm_gbs": round(v["layer_hbm_gbs"], 1),
                     "layer_hbm_frac": round(v["layer_hbm_gbs"] / HBM_PEAK_GBS, 4),
                     "layer_fp4_tflops": round(v["layer_fp4_tflops"], 1),
                     "layer_fp4_frac": round(v["layer_fp4_tflops"] / FP4_PEAK_TFLOPS, 4),
                     "gate_up_gbs": round(v["gate_up_gbs"], 1), "gate_up_tflops": round(v["gate_up_tflops"], 1),
                     "stage_us": {s: round(x * 1e3, 2) for s, x in v["stage_ms"].items()},
                     "distinct_experts": v["distinct_experts"]} for k, v in legs.items()},
    }
    if ep is not None:
        line["legs"]["prefill_t4604_zipf_ep8"] = {
            "workload": ep["workload"], "pairs": ep["pairs"], "pair_share": round(ep["pair_share"], 4),
            "experts_used": ep["experts_used"], "ms_per_step": round(ep["ms_per_step"], 5),
            "pairs_per_s": round(ep["pairs_per_s"], 1), "fp4_tflops": round(ep["fp4_tflops"], 1),
            "fp4_frac": round(ep["fp4_tflops"] / FP4_PEAK_TFLOPS, 4), "hbm_gbs": round(ep["hbm_gbs"], 1)}
    if stack is not None:
        line["legs"]["stack43_decode_t32"] = {
            "tokens_per_s": round(stack["tokens_per_s"], 1), "ms_per_step": round(stack["ms_per_step"], 4),
            "layers": stack["layers"], "hbm_gbs": round(stack["hbm_gbs"], 1),
            "hbm_frac": round(stack["hbm_gbs"] / HBM_PEAK_GBS, 4),
            "graph_tokens_per_s": round(stack["graph_tokens_per_s"], 1),
            "graph_ms_per_step": round(stack["graph_ms_per_step"], 4),
            "graph_hbm_frac": round(stack["graph_hbm_gbs"] / HBM_PEAK_GBS, 4),
            "distinct_experts_per_layer": stack["distinct_experts_per_layer"],
            "host_enqueue_ms_per_step": round(stack["host_enqueue_ms"], 3)}
    print(json.dumps(line))


if __name__ == "__main__":
    main()
