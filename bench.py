#!/usr/bin/env python3
"""Benchmark of the MoE-layer forward hot path on one MI355X.

Headline: MoE-layer microseconds per call at T=16 decode on the DeepSeek-R1 shape
(E=256, topk=8, D=7168, I=2048, bf16, BLOCK_M=16, atomic combine).  One step is one
moe_forward call -- routing (top-k softmax + sort), gate-up GEMM with SiLU-mul, down
GEMM with the routed weight, combine -- on inputs already resident in HBM.  Eight
input sets (logits and activations) rotate so the active experts change call to call.
The expert weights are put in MFMA fragment order once before timing
(moe_preshuffle_weights, the one-time weight preparation a serving process does at load);
--natural-weights times them in their [E, N, K] layout, which is also a secondary line.

The JSON line also carries the roofline of the dominant kernel (HIP events on the
stream it runs on), the CPU oracle's time on a bounded sample, and (unless
--headline-only) secondary lines: GPT-OSS decode/prefill and Kimi fp8 layer times
with per-GEMM TFLOPS, the DeepSeek and Kimi layers again with packed bf16 atomics into
the output, the Kimi shape in mxfp4 (a4w4), the Kimi prefill with the reduce-mode combine
(per-slot rows summed by the finalize kernel) instead of atomics, the headline in the other
weight layout, the DeepSeek shape at T=1 and T=4 and the other decode lines with the weights in
fragment order, router-only GB/s at T=8192 (forward and
backward), the group-limited router at the DeepSeek-V3 routing shape, and the auxiliary-loss
scores forward and backward at T=8192.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import tempfile
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0                                # MI355X HBM3E
# fp32 atomic adds to HBM-resident memory on MI355X: torch's index_add_ reaches 0.28 G adds/ms
# (--atomic-floor), this library's atomic combine 0.32 and a plain atomic-add stream 0.32-0.34
# whatever the lane pattern or occupancy; the floor of atomic mode takes 0.33
ATOMIC_ADDS_PER_S = 3.3e11
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "mxfp4": 10100.0}   # dense


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="deepseek", choices=["deepseek", "gptoss", "kimi", "kimi_mxfp4", "tiny"])
    ap.add_argument("--T", type=int, default=16)
    ap.add_argument("--rotate", type=int, default=8)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--headline-only", action="store_true", help="skip the secondary lines")
    ap.add_argument("--lines", default="layers,decode,router,grouped,aux",
                    help="secondary line groups to run (comma list of layers, decode, router, grouped, aux)")
    ap.add_argument("--natural-weights", action="store_true",
                    help="headline with the weights in their natural [E, N, K] layout instead of "
                         "fragment order (moe_preshuffle_weights, applied once before timing)")
    ap.add_argument("--details", default=os.path.join(tempfile.gettempdir(), "moe_bench_details.json"),
                    help="file for the full per-line results (the stdout line carries the headline, "
                         "its roofline, the CPU baseline and a summary); empty to skip")
    ap.add_argument("--mode", default=None, choices=["atomic", "reduce", "atomic_bf16", "reduce_bf16"],
                    help="output mode of the headline layer (default: the workload's own)")
    ap.add_argument("--atomic-floor", action="store_true",
                    help="only measure the chip's fp32 atomic-add rate (a plain stream of atomic adds "
                         "into a 470 MB buffer, torch's index_add_) and exit")
    ap.add_argument("--sequence", default=None,
                    help="only time these layer lines one after another in this process, weights in fragment "
                         "order (comma list of workload:T[:rotating sets], e.g. kimi:64:2,deepseek:4:8,kimi:64:2), "
                         "one JSON line each, and exit; a line's time can depend on what ran before it")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run a 1 GiB device copy first (counter calibration under rocprofv3 --pmc)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def graph_ms_per_call(torch, calls, n, reps=5, warm_s=0.25):
    """ms per call of `calls(i, stream)` for i in range(n), captured back to back in one HIP
    graph and replayed (median over `reps` timed replays, after `warm_s` seconds of untimed
    ones).  Host launch cost is excluded, as in the
    graph-replay measurement of the mxfp4 page ("Measurement").  Falls back to eager launches
    if the capture fails."""
    stream = torch.cuda.current_stream()
    for i in range(min(n, 3)):
        calls(i, stream)
    torch.cuda.synchronize()
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cs = torch.cuda.current_stream()
            for i in range(n):
                calls(i, cs)
        g.replay()
        torch.cuda.synchronize()
        # untimed replays first, so that the timed replays do not start while the GPU clocks
        # are still coming up from the idle host-side set-up
        t_end = time.perf_counter() + warm_s
        while time.perf_counter() < t_end:
            g.replay()
            torch.cuda.synchronize()
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) / n)
        del g
        return sorted(times)[len(times) // 2], "hip-graph"
    except Exception as exc:  # pragma: no cover - capture not available
        log(f"graph capture failed ({exc}); timing eager launches")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n):
            calls(i, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n, "eager"


def algorithmic(wl, T, n_act, num_valid):
    """Bytes and FLOPs the method must move/compute (padding, fp32 accumulator traffic,
    weight re-reads and atomic read-modify-writes excluded)."""
    E, k, D, I, B = wl.E, wl.topk, wl.D, wl.I, wl.block_m

    def nbytes(elems):  # storage of `elems` values; mxfp4: half a byte + one scale byte per 32
        return elems * 2 if wl.dtype == "bf16" else elems if wl.dtype == "fp8" else elems * 17 // 32
    route = 4 * T * E + 8 * T * k + 4 * num_valid + 4 * (num_valid // B) + 4
    g1 = nbytes(n_act * 2 * I * D) + nbytes(T * D) + nbytes(T * k * I)
    g2 = nbytes(n_act * D * I) + nbytes(T * k * I) + 4 * T * k + 2 * T * D
    if wl.dtype == "fp8":
        g1 += n_act * 2 * I * 4 + 4 * T + 4 * T * k
        g2 += n_act * D * 4 + 4 * T * k
    return {"route": route, "gemm1": g1, "gemm2": g2,
            "gemm1_flops": 2 * T * k * 2 * I * D, "gemm2_flops": 2 * T * k * D * I}


def measure_layer(env, wl, T, steps, warmup, rotate, mode=None, preshuffled=False):
    """Times moe_forward and, separately, each stage; returns a result dict.  mode overrides
    the workload's output mode (atomic_bf16: packed bf16 atomics straight into out);
    preshuffled puts the weights in fragment order first (a one-time step, not timed)."""
    m, torch, np, synth, dev = env
    k, B, dtype = wl.topk, wl.block_m, wl.dtype
    mode = mode or wl.mode
    E, D, I = wl.E, wl.D, wl.I
    log(f"{wl.name} T={T} E={E} k={k} D={D} I={I} B={B} {dtype} {mode}"
        f"{' preshuffled' if preshuffled else ''}: generating inputs")
    base = synth.layer_inputs(wl, 1, seed=0, device=dev)
    # the weights the GPU calls read (base keeps the natural layout for the CPU oracle)
    gw = {key: base.get(key) for key in ("w1", "w2", "w1_scale", "w2_scale")}
    if preshuffled:
        for key in ("w1", "w2"):
            gw[key] = m.moe_preshuffle_weights(dtype, base[key])
        if dtype == "mxfp4":  # the E8M0 block scales go into fragment order with their weights
            for key in ("w1_scale", "w2_scale"):
                gw[key] = m.moe_preshuffle_scales(base[key])
        torch.cuda.synchronize()
    pre = dict(preshuffled=True) if preshuffled else {}
    sets = []
    for r in range(rotate):
        s = {"logits": synth.logits(T, E, seed=100 + r).to(dev)}
        s.update({kk: v.to(dev) for kk, v in synth.activations(T, D, dtype, seed=100 + r, x_std=wl.x_std).items()})
        sets.append(s)
    total, offs = m.moe_forward_workspace_layout(dtype, mode, T, E, k, D, I, B)
    ws = torch.empty(total, dtype=torch.uint8, device=dev)
    out = torch.empty(T, D, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    def layer_call(i, st):
        s = sets[i % len(sets)]
        m.moe_forward(dtype, s["logits"], s["x"], gw["w1"], gw["w2"], k, B, mode,
                      x_scale=s.get("x_scale"), w1_scale=gw["w1_scale"],
                      w2_scale=gw["w2_scale"], workspace=ws, out=out, stream=st, **pre)

    for i in range(warmup):
        layer_call(i, stream)
    torch.cuda.synchronize()
    log(f"timing {steps} moe_forward calls (graph replay)")
    # a full second of untimed replays: the whole-layer graph is the first GPU work after the
    # host-side input set-up, and a quarter second left it reading up to 3% slow
    ms_per_call, how = graph_ms_per_call(torch, layer_call, steps, warm_s=1.0)

    # per-stage durations: each stage alone, `steps` calls per graph, on per-set routing
    views = m.workspace_views(ws, offs, dtype, mode, T, E, k, D, I, B)
    a, a_scale, y = views["a"], views["a_scale"], views["y"]
    if mode == "atomic_bf16":
        y = out  # stage 2 adds into the bf16 output (the timing leaves its values meaningless)
    g1ws = ws[offs["gemm1_scratch"]:] if offs["gemm1_scratch"] is not None else None
    rws = ws[offs["route_scratch"]:] if offs["route_scratch"] is not None else None
    routes, per_set = [], []
    for s in sets:  # routing of each input set into its own buffers; active experts (untimed)
        r = m.moe_topk_softmax_sort(s["logits"], k, B, workspace=rws, stream=stream)
        torch.cuda.synchronize()
        routes.append(r)
        per_set.append((len(np.unique(r["topk_ids"].cpu().numpy())), int(r["num_valid"].item())))

    def route_call(i, st):
        j = i % len(sets)
        m.moe_topk_softmax_sort(sets[j]["logits"], k, B, out=routes[j], workspace=rws, stream=st)

    def gemm1_call(i, st):
        j = i % len(sets)
        m.moe_gemm1_gateup(dtype, sets[j]["x"], gw["w1"], routes[j], k, B, x_scale=sets[j].get("x_scale"),
                           w1_scale=gw["w1_scale"], a=a, a_scale=a_scale, workspace=g1ws, stream=st,
                           **pre)

    def gemm2_call(i, st):
        j = i % len(sets)
        m.moe_gemm2_down(dtype, a, gw["w2"], routes[j], T, k, B, mode, a_scale=a_scale,
                         w2_scale=gw["w2_scale"], y=y, stream=st, **pre)

    def fin_call(i, st):
        m.moe_finalize(mode, y, T, k, D, out=out, stream=st)

    stage_ms = {}
    stages = [("route", route_call), ("gemm1", gemm1_call), ("gemm2", gemm2_call)]
    if mode != "atomic_bf16":  # packed bf16 atomics: stage 2 wrote out, no combine launch
        stages.append(("finalize", fin_call))
    for name, fn in stages:
        stage_ms[name], _ = graph_ms_per_call(torch, fn, steps)
    acc = {"route": 0, "gemm1": 0, "gemm2": 0, "gemm1_flops": 0, "gemm2_flops": 0}
    n_acts = []
    for i in range(steps):
        n_act, nv = per_set[i % len(sets)]
        n_acts.append(n_act)
        for key, v in algorithmic(wl, T, n_act, nv).items():
            acc[key] += v
    per = {key: v / steps for key, v in acc.items()}
    layer_bytes = per["route"] + per["gemm1"] + per["gemm2"]
    gemm = {}
    for g in ("gemm1", "gemm2"):
        t_s = stage_ms[g] / 1e3
        gbs = per[g] / t_s / 1e9
        tflops = per[g + "_flops"] / t_s / 1e12
        t_hbm = per[g] / (HBM_PEAK_GBS * 1e9)
        t_mfma = per[g + "_flops"] / (MFMA_PEAK_TFLOPS[dtype] * 1e12)
        gemm[g] = {"us": round(stage_ms[g] * 1e3, 2), "alg_bytes": int(per[g]), "GB/s": round(gbs, 1),
                   "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "TFLOPS": round(tflops, 1),
                   "mfma_frac": round(tflops / MFMA_PEAK_TFLOPS[dtype], 4),
                   "binding": "hbm" if t_hbm >= t_mfma else "mfma",
                   "frac_of_binding_floor": round(max(t_hbm, t_mfma) / t_s, 4)}
    if mode in ("atomic", "atomic_bf16"):
        # one fp32 atomic add per slot and model_dim channel, or one packed bf16 add per
        # channel pair; the floor takes the measured fp32 rate for both (the packed rate is
        # assumed equal, per 32-bit operation)
        adds = T * k * D if mode == "atomic" else T * k * D // 2
        gemm["gemm2"]["atomic_adds"] = adds
        gemm["gemm2"]["atomic_floor_us"] = round(adds / ATOMIC_ADDS_PER_S * 1e6, 1)
        gemm["gemm2"]["frac_of_atomic_floor"] = round(adds / ATOMIC_ADDS_PER_S / (stage_ms["gemm2"] / 1e3), 4)
    res = {
        "workload": wl.name, "T": T, "dtype": dtype, "mode": mode,
        "weights": "fragment order" if preshuffled else "natural", "us_per_call": round(ms_per_call * 1e3, 2),
        "timing": how,
        "layer_alg_bytes": int(layer_bytes), "layer_hbm_floor_us": round(layer_bytes / HBM_PEAK_GBS / 1e3, 1),
        "frac_of_layer_hbm_floor": round(layer_bytes / HBM_PEAK_GBS / 1e3 / (ms_per_call * 1e3), 4),
        "mean_active_experts": round(float(np.mean(n_acts)), 1),
        "stage_us": {kk: round(v * 1e3, 2) for kk, v in stage_ms.items()},
        "route_GB/s": round(per["route"] / (stage_ms["route"] / 1e3) / 1e9, 1),
        "gemm": gemm,
    }
    keep = (base, sets)
    return res, keep


def measure_router(env, E, k, score, steps, warmup):
    """Router-only (top-k + sort) at T = 8192, BLOCK_M = 32, input sets rotated past the
    256 MB last-level cache."""
    m, torch, np, synth, dev = env
    T, B = synth.ROUTER_T, synth.ROUTER_BLOCK_M
    R = max(2, -(-512 * 2**20 // (4 * T * E)))
    sets = [synth.logits(T, E, seed=200 + r).to(dev) for r in range(R)]
    cap = m.moe_sorted_capacity(T, E, k, B)
    rt = {"topk_weights": torch.empty(T, k, device=dev), "topk_ids": torch.empty(T, k, dtype=torch.int32, device=dev),
          "sorted_token_ids": torch.empty(cap, dtype=torch.int32, device=dev),
          "expert_ids": torch.empty(cap // B, dtype=torch.int32, device=dev),
          "num_valid": torch.empty(1, dtype=torch.int32, device=dev)}
    nb = m.moe_route_workspace_bytes(T, E, k, B)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    def call(i, st):
        m.moe_topk_softmax_sort(sets[i % R], k, B, score, out=rt, workspace=ws, stream=st)

    for i in range(warmup):
        call(i, stream)
    torch.cuda.synchronize()
    nv = int(rt["num_valid"].item())
    ms, how = graph_ms_per_call(torch, call, max(steps, R))
    us = ms * 1e3
    alg = 4 * T * E + 8 * T * k + 4 * nv + 4 * (nv // B) + 4
    gbs = alg / (us * 1e-6) / 1e9
    res = {"router": f"{E}/{k}", "score": score, "T": T, "block_m": B, "us_per_call": round(us, 2),
           "alg_bytes": alg, "GB/s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
           "rotating_input_sets": R, "timing": how}

    # backward of the weights at each set's picks: reads the picks' ids, weights and weight
    # gradients (sigmoid: also the picked logits), writes the dense [T, E] logit gradient
    picks = []
    for r in range(R):
        m.moe_topk_softmax_sort(sets[r], k, B, score, out=rt, workspace=ws, stream=stream)
        picks.append((rt["topk_ids"].clone(), rt["topk_weights"].clone()))
    gw = torch.randn(T, k, device=dev)
    gl = torch.empty(T, E, device=dev)

    def bwd(i, st):
        ids, w = picks[i % R]
        m.moe_topk_softmax_backward(sets[i % R], ids, w, gw, score, True, grad_logits=gl, stream=st)

    for i in range(warmup):
        bwd(i, stream)
    torch.cuda.synchronize()
    ms_b, _ = graph_ms_per_call(torch, bwd, max(steps, R))
    alg_b = 4 * T * E + 12 * T * k + (4 * T * k if score == "sigmoid" else 0)
    gbs_b = alg_b / (ms_b * 1e-3) / 1e9
    res["backward"] = {"us_per_call": round(ms_b * 1e3, 2), "alg_bytes": alg_b, "GB/s": round(gbs_b, 1),
                       "hbm_frac": round(gbs_b / HBM_PEAK_GBS, 4)}
    return res


def measure_router_grouped(env, T, E, k, n_group, topk_group, score, B, steps, warmup):
    """Group-limited router (top-k over the best topk_group of n_group expert groups, then the
    sort) at the DeepSeek-V3 routing shape, beside the plain router on the same inputs."""
    m, torch, np, synth, dev = env
    R = min(256, max(4, -(-512 * 2**20 // (4 * T * E))))
    sets = [synth.logits(T, E, seed=300 + r).to(dev) for r in range(R)]
    cap = m.moe_sorted_capacity(T, E, k, B)
    rt = {"topk_weights": torch.empty(T, k, device=dev), "topk_ids": torch.empty(T, k, dtype=torch.int32, device=dev),
          "sorted_token_ids": torch.empty(cap, dtype=torch.int32, device=dev),
          "expert_ids": torch.empty(cap // B, dtype=torch.int32, device=dev),
          "num_valid": torch.empty(1, dtype=torch.int32, device=dev)}
    nb = m.moe_route_workspace_bytes(T, E, k, B)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def grouped(i, st):
        m.moe_topk_softmax_sort_grouped(sets[i % R], k, n_group, topk_group, B, score, True, out=rt,
                                        workspace=ws, stream=st)

    def plain(i, st):
        m.moe_topk_softmax_sort(sets[i % R], k, B, score, True, out=rt, workspace=ws, stream=st)

    res = {"router_grouped": f"{E}/{k}, {n_group} groups, keep {topk_group}", "score": score, "T": T,
           "block_m": B, "rotating_input_sets": R}
    for name, fn in (("grouped", grouped), ("plain", plain)):
        for i in range(warmup):
            fn(i, stream)
        torch.cuda.synchronize()
        ms, how = graph_ms_per_call(torch, fn, max(steps, R))
        res[f"{name}_us_per_call"] = round(ms * 1e3, 2)
        res["timing"] = how
    nv = int(rt["num_valid"].item())
    alg = 4 * T * E + 8 * T * k + 4 * nv + 4 * (nv // B) + 4
    res["alg_bytes"] = alg
    res["GB/s"] = round(alg / (res["grouped_us_per_call"] * 1e-6) / 1e9, 1)
    return res


def measure_aux(env, E, k, score, steps, warmup):
    """Auxiliary-loss scores at T = 8192 (the pages' router benchmark size), forward (scores
    and routing map) and backward, input sets rotated past the last-level cache."""
    m, torch, np, synth, dev = env
    T = synth.ROUTER_T
    R = max(2, -(-512 * 2**20 // (4 * T * E)))
    sets = [synth.logits(T, E, seed=400 + r).to(dev) for r in range(R)]
    sc = torch.empty(T, E, device=dev)
    rmap = torch.empty(T, E, dtype=torch.bool, device=dev)
    g = torch.randn(T, E, device=dev)
    gl = torch.empty(T, E, device=dev)
    stream = torch.cuda.current_stream()

    def fwd(i, st):
        m.moe_aux_loss_scores(sets[i % R], k, score, scores=sc, routing_map=rmap, stream=st)

    def bwd(i, st):
        m.moe_aux_loss_scores_backward(sets[i % R], g, score, grad_logits=gl, stream=st)

    res = {"aux_scores": f"{E}/{k}", "score": score, "T": T, "rotating_input_sets": R}
    # forward: logits in, scores and map out (9 B per element); backward: logits and the
    # score gradient in, logit gradient out (12 B per element)
    for name, fn, per in (("forward", fwd, 9), ("backward", bwd, 12)):
        for i in range(warmup):
            fn(i, stream)
        torch.cuda.synchronize()
        ms, how = graph_ms_per_call(torch, fn, max(steps, R))
        alg = per * T * E
        gbs = alg / (ms * 1e-3) / 1e9
        res[name] = {"us_per_call": round(ms * 1e3, 2), "alg_bytes": alg, "GB/s": round(gbs, 1),
                     "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "timing": how}
    return res


KERNEL_SOURCES = ("mixture_experts_routing_amd/csrc/gemm.hip", "mixture_experts_routing_amd/csrc/moe_device.h")


def achievable_peaks(torch, dev):
    """What PyTorch's own kernels reach on this GPU, reported beside the spec-sheet peaks as
    context (not as a ceiling: the layer's gemm1 streams faster than torch's sum reads): a
    streaming read (sum over 4 GiB), a device copy (1 GiB each way, both directions counted),
    and dense 8192^3 matmuls (bf16, and fp8 e4m3 with unit scales when torch supports it)."""
    res = {}
    def timed(fn, n=10):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n / 1e3
    a = torch.empty(1 << 30, dtype=torch.float32, device=dev)
    a.fill_(1.0)
    res["hbm_read_GBps"] = round(4 * 2**30 / timed(lambda: a.sum()) / 1e9, 1)
    del a
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    res["hbm_copy_GBps"] = round(2 * 2**30 / timed(lambda: dst.copy_(src)) / 1e9, 1)
    del src, dst
    n = 8192
    x = torch.randn(n, n, device=dev).to(torch.bfloat16)
    y = torch.randn(n, n, device=dev).to(torch.bfloat16)
    res["bf16_matmul_TFLOPS"] = round(2 * n**3 / timed(lambda: x @ y) / 1e12, 1)
    try:
        xf = x.to(torch.float8_e4m3fn)
        yf = y.t().contiguous().to(torch.float8_e4m3fn).t()
        one = torch.ones((), device=dev)
        res["fp8_matmul_TFLOPS"] = round(
            2 * n**3 / timed(lambda: torch._scaled_mm(xf, yf, scale_a=one, scale_b=one, out_dtype=torch.bfloat16)) / 1e12, 1)
    except Exception as exc:  # pragma: no cover - depends on the torch build
        res["fp8_matmul_TFLOPS"] = None
        res["fp8_matmul_note"] = f"torch._scaled_mm unavailable: {type(exc).__name__}"
    del x, y
    torch.cuda.empty_cache()
    return res


def atomic_floor(torch, dev):
    """fp32 atomic adds per second into HBM-resident memory: torch's index_add_ adds a
    [n, 7168] fp32 source into a [16384, 7168] destination (470 MB, the Kimi-K2.5 T=16384
    accumulator) through rows chosen at random, one atomic add per element, timed over
    graph-free eager launches.  Two lane patterns: whole rows (64 consecutive floats per
    wave instruction) and the same adds with the destination rows in a random permutation."""
    T, D = 16384, 7168
    y = torch.zeros(T, D, device=dev)
    n = 147456 // 4  # a quarter of the Kimi T=16384 slot rows per launch
    src = torch.randn(n, D, device=dev)
    res = {"destination_MB": round(T * D * 4 / 1e6, 1), "adds_per_launch": n * D}
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    for name, idx in (("rows_in_order", torch.arange(n, device=dev) % T),
                      ("rows_random", torch.randint(0, T, (n,), device=dev, generator=g))):
        for _ in range(3):
            y.index_add_(0, idx, src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        e0.record()
        for _ in range(reps):
            y.index_add_(0, idx, src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res[name] = {"ms_per_launch": round(ms, 3), "G_adds_per_ms": round(n * D / ms / 1e9, 4)}
    return res


def kernel_source_sha256():
    """sha256 of the GEMM sources with comments and blank space removed, so that only code
    changes (which can change the kernels' traffic) invalidate stored counter readings."""
    import hashlib
    import re
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        src = re.sub(r"//[^\n]*", "", src)
        h.update("".join(src.split()).encode())
    return h.hexdigest()


def pmc_traffic(kernel, wl, T):
    """HBM bytes per launch of `kernel` from the committed counter summary for this workload
    (FETCH_SIZE and WRITE_SIZE, each scaled by a plain copy's reading), or None when there is
    none or the GEMM sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{wl.name}_T{T}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.split(":", 1)[0].strip() in ("traffic_bytes_per_launch", "source_sha256"):
                key, val = line.split(":", 1)
                fields[key.strip()] = val.strip().strip("`")
    if fields.get("source_sha256") != kernel_source_sha256():
        return None
    return int(fields["traffic_bytes_per_launch"]) if "traffic_bytes_per_launch" in fields else None


def cpu_baseline(env, wl, T, keep, n_calls=3):
    """The CPU oracle on whole calls of the headline workload (routing of all T tokens and the
    layer for every token, fp64 numpy), one call per input set for the first n_calls sets, timed
    on the host cores; the value is the mean per call.  Expert weights are copied to host memory
    before the clock starts; only what the calls read is copied."""
    m, torch, np, synth, dev = env
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    base, sets = keep
    hb = lambda t: t.detach().cpu().view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.detach().cpu().numpy()  # noqa: E731
    calls = []
    used = set()
    for s in sets[:n_calls]:
        host_logits = s["logits"].cpu().numpy()
        host_x = hb(s["x"])
        host_xs = s["x_scale"].cpu().numpy() if "x_scale" in s else None
        r = oracle.route(host_logits, wl.topk, wl.block_m)
        used |= set(r.ids.reshape(-1).tolist())
        calls.append((host_logits, host_x, host_xs))
    used = sorted(used)
    W1 = {e: hb(base["w1"][e]) for e in used}
    W2 = {e: hb(base["w2"][e]) for e in used}
    W1s = {e: base["w1_scale"][e].cpu().numpy() for e in used} if "w1_scale" in base else None
    W2s = {e: base["w2_scale"][e].cpu().numpy() for e in used} if "w2_scale" in base else None
    t0 = time.perf_counter()
    for host_logits, host_x, host_xs in calls:
        r = oracle.route(host_logits, wl.topk, wl.block_m)
        oracle.moe_layer(host_x, W1, W2, r.ids, r.weights, wl.dtype, x_scale=host_xs, w1_scale=W1s,
                         w2_scale=W2s)
    dt = time.perf_counter() - t0
    del W1, W2
    n = len(calls)
    return {"value": round(dt / n * 1e6, 1), "unit": "us/call", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": (f"{n} whole {wl.name} T={T} calls (input sets 0..{n - 1}): routing of all {T} tokens and "
                       f"the layer for all {T} tokens of each, {len(used)} distinct active experts, fp64 numpy, "
                       f"{dt:.2f} s in total; BLAS threads {blas_threads}, host logical CPUs {os.cpu_count()}")}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): this library has no multi-GPU "
              "path", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import mixture_experts_routing_amd as m
    import synth

    m.load_library()
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    env = (m, torch, np, synth, dev)
    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    wl = synth.WORKLOADS[args.workload]
    if args.atomic_floor:
        print(json.dumps(atomic_floor(torch, dev)), flush=True)
        return
    if args.sequence:
        for item in args.sequence.split(","):
            name, T, *rot = item.split(":")
            r, kp = measure_layer(env, synth.WORKLOADS[name], int(T), args.steps, args.warmup,
                                  int(rot[0]) if rot else args.rotate, None, preshuffled=True)
            del kp
            torch.cuda.empty_cache()
            print(json.dumps({"line": item, "us_per_call": r["us_per_call"], "stage_us": r["stage_us"],
                              "stage_sum_us": round(sum(r["stage_us"].values()), 2)}), flush=True)
        return
    head, keep = measure_layer(env, wl, args.T, args.steps, args.warmup, args.rotate, args.mode,
                               preshuffled=not args.natural_weights)
    g1 = head["gemm"]["gemm1"]
    g2 = head["gemm"]["gemm2"]
    dom_name, dom = max((("gemm1", g1), ("gemm2", g2)), key=lambda kv: kv[1]["us"])
    if dom["binding"] == "hbm":
        roofline = {"bound": "hbm", "achieved": dom["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": dom["hbm_frac"], "traffic": None}
    else:
        roofline = {"bound": "mfma", "achieved": dom["TFLOPS"], "peak": MFMA_PEAK_TFLOPS[wl.dtype],
                    "unit": "TFLOP/s", "frac": dom["mfma_frac"], "traffic": None}
    roofline["traffic"] = pmc_traffic(dom_name, wl, args.T)
    roofline.update(kernel=f"{dom_name}_kernel", avg_launch_us=dom["us"], alg_bytes_per_launch=dom["alg_bytes"])

    cpu = None
    if not args.no_cpu:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(env, wl, args.T, keep)
    del keep
    torch.cuda.empty_cache()

    log("measuring achievable peaks (torch streaming read, copy, dense matmuls)")
    peaks = achievable_peaks(torch, dev)

    secondary = []

    def emit(r):
        secondary.append(r)
        log(brief(r))

    groups = set() if args.headline_only else set(args.lines.split(","))
    if "layers" in groups:
        for name, T, mode in (("gptoss", 16, None), ("gptoss", 4096, None), ("kimi", 64, None),
                              ("kimi", 4096, None), ("kimi", 16384, None), ("deepseek", 16, "atomic_bf16"),
                              ("kimi", 4096, "atomic_bf16"), ("kimi", 16384, "atomic_bf16"),
                              ("kimi_mxfp4", 64, None), ("kimi_mxfp4", 4096, None),
                              ("kimi_mxfp4", 16384, None), ("kimi", 4096, "reduce"),
                              ("kimi", 16384, "reduce"), ("kimi_mxfp4", 16384, "reduce"),
                              ("gptoss", 4096, "reduce_bf16"), ("kimi", 4096, "reduce_bf16"),
                              ("kimi", 16384, "reduce_bf16"), ("kimi_mxfp4", 16384, "reduce_bf16")):
            r, kp = measure_layer(env, synth.WORKLOADS[name], T, max(5, args.steps // 2), 2, 2, mode)
            del kp
            torch.cuda.empty_cache()
            emit(r)
    if "decode" in groups:
        # the headline with the other weight layout, and the decode lines in fragment order
        # (prepared once, outside the timed region)
        for name, T, pre in ((args.workload, args.T, args.natural_weights), ("deepseek", 1, True),
                             ("deepseek", 2, True), ("deepseek", 4, True), ("deepseek", 8, True), ("kimi", 64, True),
                             ("kimi_mxfp4", 64, True),
                             ("gptoss", 16, True)):
            # input sets rotated as in the natural-layout line of the same workload
            rot = args.rotate if name == args.workload or name == "deepseek" else 2
            r, kp = measure_layer(env, synth.WORKLOADS[name], T, max(5, args.steps // 2), 2, rot, None,
                                  preshuffled=pre)
            del kp
            torch.cuda.empty_cache()
            emit(r)
    if "router" in groups:
        for (E, k) in synth.ROUTER_CASES:
            for score in ("softmax", "sigmoid"):
                emit(measure_router(env, E, k, score, args.steps, 3))
        torch.cuda.empty_cache()
    if "grouped" in groups:
        for T, B in ((16, 16), (synth.ROUTER_T, synth.ROUTER_BLOCK_M)):
            emit(measure_router_grouped(env, T, 256, 8, 8, 4, "sigmoid", B, args.steps, 3))
    if "aux" in groups:
        for (E, k) in synth.AUX_CASES:
            for score in ("softmax", "sigmoid"):
                emit(measure_aux(env, E, k, score, args.steps, 3))
        torch.cuda.empty_cache()

    details = {"layer": head, "achievable_peaks": peaks, "secondary": secondary}
    if args.details:
        os.makedirs(os.path.dirname(os.path.abspath(args.details)), exist_ok=True)
        with open(args.details, "w") as f:
            json.dump(details, f, indent=1)
        log(f"full results written to {args.details}")
    print(record_line(args, wl, head, roofline, cpu, secondary), flush=True)


def record_line(args, wl, head, roofline, cpu, secondary):
    """The one JSON line the run ends with (kept under 4000 characters): the headline, its
    roofline, the CPU baseline, the headline's stage times and a summary of the secondary
    lines.  The full per-line results go to the --details file."""
    res = {
        "metric": f"moe_layer_us_per_call_T{args.T}_decode" if args.workload == "deepseek"
        else f"moe_layer_us_per_call_{wl.name}_T{args.T}",
        "value": head["us_per_call"],
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["us_per_call"] / 1e3, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": f"{wl.name}-shaped MoE layer forward, T={args.T}", "T": args.T, "E": wl.E,
                   "topk": wl.topk, "D": wl.D, "I": wl.I, "block_m": wl.block_m, "mode": head["mode"],
                   "rotating_input_sets": args.rotate,
                   "weights": "natural" if args.natural_weights else "fragment order (prepared once)"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "stage_us": head["stage_us"],
        "layer_frac_of_hbm_floor": head["frac_of_layer_hbm_floor"],
        "summary": summarize(secondary) if secondary else None,
    }
    line = json.dumps(res, separators=(",", ":"))
    if len(line) > 4000:  # keep the record one short line: the summary goes first
        res["summary"] = None
        line = json.dumps(res, separators=(",", ":"))
    return line


def summarize(secondary):
    """The other two parts of the metric, from the secondary lines: prefill GEMM TFLOPS with
    their fraction of the dense MFMA peak (and of the binding floor), routing GB/s with their
    fraction of HBM peak, and the other decode layer times (weights in fragment order)."""
    import synth
    out = {"prefill": {}, "router": {}, "decode": {}}
    for r in secondary:
        if "workload" in r:
            default_mode = r["mode"] == synth.WORKLOADS[r["workload"]].mode
            key = f"{r['workload']}_T{r['T']}" + ("" if default_mode else f"_{r['mode']}")
            if r["T"] >= 1024:
                g1, g2 = r["gemm"]["gemm1"], r["gemm"]["gemm2"]
                out["prefill"][key] = {
                    "us": r["us_per_call"],
                    "gemm1": [g1["us"], g1["TFLOPS"], g1["mfma_frac"], g1["frac_of_binding_floor"]],
                    "gemm2": [g2["us"], g2["TFLOPS"], g2["mfma_frac"], g2["frac_of_binding_floor"]]}
            elif default_mode and r["weights"] == "fragment order":
                out["decode"][key] = [r["us_per_call"], r["frac_of_layer_hbm_floor"]]
        elif "router" in r:
            out["router"][f"{r['router']}_{r['score']}"] = [r["us_per_call"], r["GB/s"], r["hbm_frac"]]
    out["legend"] = {"prefill": "gemm1/gemm2: [us, TFLOPS, frac of dense MFMA peak, frac of binding floor]",
                     "router": "[us, GB/s, frac of HBM peak], T=8192",
                     "decode": "[us/call, frac of layer HBM floor]"}
    return out


def brief(r):
    """One short line describing a secondary result (progress on stderr)."""
    if "workload" in r:
        return (f"{r['workload']} T={r['T']} {r['mode']} {r['weights']}: {r['us_per_call']} us "
                f"(stages {r['stage_us']})")
    if "router" in r:
        return f"router {r['router']} {r['score']}: {r['us_per_call']} us, {r['GB/s']} GB/s"
    if "router_grouped" in r:
        return f"grouped router T={r['T']}: {r['grouped_us_per_call']} us"
    return f"aux scores {r['aux_scores']} {r['score']}: fwd {r['forward']['us_per_call']} us"


if __name__ == "__main__":
    main()
