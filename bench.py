#!/usr/bin/env python3
"""Benchmark of the MoE-layer forward hot path on one MI355X.

Headline: MoE-layer microseconds per call at T=16 decode on the DeepSeek-R1 shape
(E=256, topk=8, D=7168, I=2048, bf16, BLOCK_M=16, atomic combine).  One step is one
moe_forward call: routing (top-k softmax + sort), gate-up GEMM, down GEMM with the
routed weight and the combine, on inputs already resident in HBM.  Eight input sets
(logits and activations) rotate so the set of active experts changes call to call.

Prints one JSON line with the metric, the roofline of the dominant kernel (timed
with HIP events on the stream it runs on) and the CPU oracle's time on a bounded
sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}  # dense


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="deepseek", choices=["deepseek", "gptoss", "kimi", "tiny"])
    ap.add_argument("--T", type=int, default=16)
    ap.add_argument("--rotate", type=int, default=8)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    return ap.parse_args()


def algorithmic(wl, T, n_act, num_valid, dtype):
    """Bytes and FLOPs the method must move/compute (padding, fp32 accumulator traffic,
    weight re-reads and atomic read-modify-writes excluded)."""
    E, k, D, I, B = wl.E, wl.topk, wl.D, wl.I, wl.block_m
    bw = 2 if dtype == "bf16" else 1
    route = 4 * T * E + 8 * T * k + 4 * num_valid + 4 * (num_valid // B) + 4
    g1 = n_act * 2 * I * D * bw + T * D * bw + T * k * I * bw
    g2 = n_act * D * I * bw + T * k * I * bw + 4 * T * k + 2 * T * D
    if dtype == "fp8":
        g1 += n_act * 2 * I * 4 + 4 * T + 4 * T * k
        g2 += n_act * D * 4 + 4 * T * k
    return {"route_bytes": route, "gemm1_bytes": g1, "gemm2_bytes": g2,
            "gemm1_flops": 2 * T * k * 2 * I * D, "gemm2_flops": 2 * T * k * D * I}


def cpu_baseline(wl, T, host_logits, host_x, host_xs, w1, w2, w1s, w2s, n_act_all):
    """The CPU oracle, timed on a bounded sample (the first tokens of one input set),
    scaled to a whole call by active-expert count (its cost is per expert read)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    sample_tokens = list(range(min(2, T)))
    r = oracle.route(host_logits, wl.topk, wl.block_m)
    used = sorted(set(r.ids[sample_tokens].reshape(-1).tolist()))
    # host copies of exactly the weights the sample reads (untimed)
    W1 = {e: w1(e) for e in used}
    W2 = {e: w2(e) for e in used}
    W1s = {e: w1s(e) for e in used} if w1s else None
    W2s = {e: w2s(e) for e in used} if w2s else None
    t0 = time.perf_counter()
    r = oracle.route(host_logits, wl.topk, wl.block_m)
    oracle.moe_layer(host_x, W1, W2, r.ids, r.weights, wl.dtype, x_scale=host_xs, w1_scale=W1s,
                     w2_scale=W2s, tokens=sample_tokens)
    dt = time.perf_counter() - t0
    per_call_us = dt * 1e6 * (n_act_all / len(used))
    return {"value": round(per_call_us, 1), "unit": "us/call", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": (f"{wl.name} T={T}: routing of all {T} tokens + layer for tokens {sample_tokens} "
                       f"({len(used)} of {n_act_all} active experts), fp64 numpy, {dt:.2f} s, "
                       f"scaled by active experts; host has {os.cpu_count()} logical CPUs")}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the path has no multi-GPU "
              "component in this build", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import mixture_experts_routing_amd as m
    import synth

    m.load_library()
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    wl = synth.WORKLOADS[args.workload]
    T, k, B, dtype, mode = args.T, wl.topk, wl.block_m, wl.dtype, wl.mode
    E, D, I = wl.E, wl.D, wl.I
    print(f"[bench] {wl.name} T={T} E={E} k={k} D={D} I={I} B={B} {dtype} {mode}: generating inputs",
          file=sys.stderr, flush=True)
    base = synth.layer_inputs(wl, 1, seed=0, device=dev)
    sets = []
    for r in range(args.rotate):
        s = {"logits": synth.logits(T, E, seed=100 + r).to(dev)}
        s.update({kk: v.to(dev) for kk, v in synth.activations(T, D, dtype, seed=100 + r, x_std=wl.x_std).items()})
        sets.append(s)
    total, offs = m.moe_forward_workspace_layout(dtype, mode, T, E, k, D, I, B)
    ws = torch.empty(total, dtype=torch.uint8, device=dev)
    out = torch.empty(T, D, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        s = sets[i % len(sets)]
        m.moe_forward(dtype, s["logits"], s["x"], base["w1"], base["w2"], k, B, mode,
                      x_scale=s.get("x_scale"), w1_scale=base.get("w1_scale"),
                      w2_scale=base.get("w2_scale"), workspace=ws, out=out, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    print(f"[bench] warmup done, timing {args.steps} steps", file=sys.stderr, flush=True)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps

    # per-stage durations (HIP events on the launch stream), staged calls on the same inputs
    views = m.workspace_views(ws, offs, dtype, mode, T, E, k, D, I, B)
    stage_ms = {"route": [], "gemm1": [], "gemm2": [], "finalize": []}
    bytes_acc = {"gemm1": 0, "gemm2": 0, "route": 0}
    flops_acc = {"gemm1": 0, "gemm2": 0}
    rt = {kk: views[kk] for kk in ("topk_weights", "topk_ids", "sorted_token_ids", "expert_ids", "num_valid")}
    a = views["a"]
    a_scale = views["a_scale"]
    y = views["y"]
    g1ws = ws[offs["gemm1_scratch"]:] if offs["gemm1_scratch"] is not None else None
    rws = ws[offs["route_scratch"]:] if offs["route_scratch"] is not None else None
    # active experts and num_valid of each input set (read back once, untimed)
    per_set = []
    for s in sets:
        m.moe_topk_softmax_sort(s["logits"], k, B, out=rt, workspace=rws, stream=stream)
        torch.cuda.synchronize()
        per_set.append((len(np.unique(rt["topk_ids"].cpu().numpy())), int(rt["num_valid"].item())))
    # all steps are enqueued before one synchronisation, so the GPU never waits on the
    # host between an event and the kernel it brackets
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    n_acts = []
    for i in range(args.steps):
        s = sets[i % len(sets)]
        ev = evs[i]
        if mode == "atomic":
            y.zero_()  # outside every bracketed interval
        ev[0].record(stream)
        m.moe_topk_softmax_sort(s["logits"], k, B, out=rt, workspace=rws, stream=stream)
        ev[1].record(stream)
        m.moe_gemm1_gateup(dtype, s["x"], base["w1"], rt, k, B, x_scale=s.get("x_scale"),
                           w1_scale=base.get("w1_scale"), a=a, a_scale=a_scale, workspace=g1ws, stream=stream)
        ev[2].record(stream)
        m.moe_gemm2_down(dtype, a, base["w2"], rt, T, k, B, mode, a_scale=a_scale,
                         w2_scale=base.get("w2_scale"), y=y, stream=stream)
        ev[3].record(stream)
        m.moe_finalize(mode, y, T, k, D, out=out, stream=stream)
        ev[4].record(stream)
        n_act, nv = per_set[i % len(sets)]
        n_acts.append(n_act)
        alg = algorithmic(wl, T, n_act, nv, dtype)
        bytes_acc["gemm1"] += alg["gemm1_bytes"]
        bytes_acc["gemm2"] += alg["gemm2_bytes"]
        bytes_acc["route"] += alg["route_bytes"]
        flops_acc["gemm1"] += alg["gemm1_flops"]
        flops_acc["gemm2"] += alg["gemm2_flops"]
    torch.cuda.synchronize()
    for ev in evs:
        for j, name in enumerate(("route", "gemm1", "gemm2", "finalize")):
            stage_ms[name].append(ev[j].elapsed_time(ev[j + 1]))
    mean_ms = {kk: float(np.mean(v)) for kk, v in stage_ms.items()}
    dominant = max(("gemm1", "gemm2"), key=lambda kk: mean_ms[kk])
    n_launch = args.steps
    dom_bytes = bytes_acc[dominant] / n_launch
    dom_s = mean_ms[dominant] / 1e3
    achieved = dom_bytes / dom_s / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": f"{dominant} ({'gemm1_kernel' if dominant == 'gemm1' else 'gemm2_kernel'})",
                "alg_bytes_per_launch": int(dom_bytes), "avg_launch_us": round(mean_ms[dominant] * 1e3, 2)}
    layer_bytes = (bytes_acc["gemm1"] + bytes_acc["gemm2"] + bytes_acc["route"]) / n_launch
    stages = {kk: round(v * 1e3, 2) for kk, v in mean_ms.items()}

    cpu = None
    if not args.no_cpu:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        s = sets[0]
        hb = lambda t: t.detach().cpu().view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.detach().cpu().numpy()  # noqa: E731
        ids0 = None
        m.moe_topk_softmax_sort(s["logits"], k, B, out=rt, workspace=rws, stream=stream)
        torch.cuda.synchronize()
        ids0 = rt["topk_ids"].cpu().numpy()
        cpu = cpu_baseline(
            wl, T, s["logits"].cpu().numpy(), hb(s["x"]),
            s["x_scale"].cpu().numpy() if "x_scale" in s else None,
            lambda e: hb(base["w1"][e]), lambda e: hb(base["w2"][e]),
            (lambda e: base["w1_scale"][e].cpu().numpy()) if "w1_scale" in base else None,
            (lambda e: base["w2_scale"][e].cpu().numpy()) if "w2_scale" in base else None,
            len(np.unique(ids0)))

    res = {
        "metric": f"moe_layer_us_per_call_T{T}_decode" if args.workload == "deepseek" else f"moe_layer_us_per_call_{wl.name}_T{T}",
        "value": round(ms_per_step * 1e3, 2),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": f"{wl.name}-shaped MoE layer forward", "T": T, "E": E, "topk": k, "D": D,
                   "I": I, "block_m": B, "mode": mode, "score": "softmax", "renorm": True,
                   "rotating_input_sets": args.rotate},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "layer": {"alg_bytes_per_call": int(layer_bytes), "hbm_floor_us": round(layer_bytes / HBM_PEAK_GBS / 1e3, 1),
                  "frac_of_hbm_floor": round(layer_bytes / HBM_PEAK_GBS / 1e3 / (ms_per_step * 1e3), 4),
                  "mean_active_experts": round(float(np.mean(n_acts)), 1), "stage_us": stages},
    }
    print(json.dumps(res))


if __name__ == "__main__":
    main()
