"""The benchmark's closing JSON line: one line under 4000 characters that carries the headline,
its roofline, the CPU baseline and the summary of every secondary line the default run makes
(a longer line is cut by readers that keep only the end of the output)."""

import json
import os
import sys
import types

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def fake_layer(name, T, mode=None, weights="natural"):
    wl = synth.WORKLOADS[name]
    g = {"us": 1234.56, "alg_bytes": 5908011417, "GB/s": 6981.23, "hbm_frac": 0.8727, "TFLOPS": 1555.5,
         "mfma_frac": 0.3111, "binding": "hbm", "frac_of_binding_floor": 0.8727}
    gemm = {"gemm1": dict(g), "gemm2": dict(g, atomic_adds=1056964608, atomic_floor_us=3202.9,
                                            frac_of_atomic_floor=0.9676)}
    return {"workload": name, "T": T, "dtype": wl.dtype, "mode": mode or wl.mode, "weights": weights,
            "us_per_call": 1284.51, "timing": "hip-graph", "layer_alg_bytes": 8981234567,
            "layer_hbm_floor_us": 1122.7, "frac_of_layer_hbm_floor": 0.8741, "mean_active_experts": 100.6,
            "stage_us": {"route": 7.41, "gemm1": 844.87, "gemm2": 428.33, "finalize": 2.41},
            "route_GB/s": 3.1, "gemm": gemm}


def default_secondaries():
    """The secondary lines of a default run, in the shapes measure_* return."""
    out = []
    for name, T, mode in (("gptoss", 16, None), ("gptoss", 4096, None), ("kimi", 64, None),
                          ("kimi", 4096, None), ("kimi", 16384, None), ("deepseek", 16, "atomic_bf16"),
                          ("kimi", 4096, "atomic_bf16"), ("kimi", 16384, "atomic_bf16"),
                          ("kimi_mxfp4", 64, None), ("kimi_mxfp4", 4096, None),
                          ("kimi_mxfp4", 16384, None), ("kimi", 4096, "reduce"),
                          ("kimi", 16384, "reduce"), ("kimi_mxfp4", 16384, "reduce"),
                          ("gptoss", 4096, "reduce_bf16"), ("kimi", 4096, "reduce_bf16"),
                          ("kimi", 16384, "reduce_bf16"), ("kimi_mxfp4", 16384, "reduce_bf16")):
        out.append(fake_layer(name, T, mode))
    for name, T in (("deepseek", 16), ("deepseek", 1), ("deepseek", 2), ("deepseek", 4), ("deepseek", 8),
                    ("kimi", 64), ("kimi_mxfp4", 64), ("gptoss", 16)):
        out.append(fake_layer(name, T, None, "fragment order"))
    for E, k in synth.ROUTER_CASES:
        for score in ("softmax", "sigmoid"):
            out.append({"router": f"{E}/{k}", "score": score, "T": 8192, "block_m": 32, "us_per_call": 22.63,
                        "alg_bytes": 17203204, "GB/s": 760.12, "hbm_frac": 0.095, "rotating_input_sets": 31,
                        "timing": "hip-graph", "backward": {"us_per_call": 5.3, "alg_bytes": 1, "GB/s": 1.0,
                                                            "hbm_frac": 0.1}})
    for T in (16, 8192):
        out.append({"router_grouped": "256/8, 8 groups, keep 4", "score": "sigmoid", "T": T, "block_m": 16,
                    "rotating_input_sets": 4, "grouped_us_per_call": 11.0, "plain_us_per_call": 7.1,
                    "timing": "hip-graph", "alg_bytes": 1, "GB/s": 1.0})
    for E, k in synth.AUX_CASES:
        for score in ("softmax", "sigmoid"):
            out.append({"aux_scores": f"{E}/{k}", "score": score, "T": 8192, "rotating_input_sets": 4,
                        "forward": {"us_per_call": 13.3}, "backward": {"us_per_call": 9.9}})
    return out


def test_record_line_is_short_and_complete():
    args = types.SimpleNamespace(T=16, workload="deepseek", steps=20, warmup=5, rotate=8, natural_weights=False)
    head = fake_layer("deepseek", 16, None, "fragment order")
    roofline = {"bound": "hbm", "achieved": 6981.2, "peak": 8000.0, "unit": "GB/s", "frac": 0.8727,
                "traffic": 5896000000, "kernel": "gemm1_kernel", "avg_launch_us": 844.87,
                "alg_bytes_per_launch": 5908011417, "timing": "hip events on the launch stream"}
    cpu = {"value": 4567890.1, "unit": "us/call", "cores": 16, "kind": "oracle",
           "sample": "3 whole deepseek T=16 calls (input sets 0..2): routing of all 16 tokens and the layer for "
                     "all 16 tokens of each, 120 distinct active experts, fp64 numpy, 13.70 s in total; "
                     "BLAS threads 16, host logical CPUs 256"}
    sec = default_secondaries()
    for r in sec:
        bench.brief(r)  # every kind of line has a progress form
    line = bench.record_line(args, synth.WORKLOADS["deepseek"], head, roofline, cpu, sec)
    assert "\n" not in line
    assert len(line) < 4000, len(line)
    rec = json.loads(line)
    for key in ("metric", "value", "unit", "ms_per_step", "steps", "dtype", "roofline", "cpu_baseline"):
        assert rec[key] is not None
    assert rec["config"]["workload"]
    summ = rec["summary"]
    assert summ is not None
    assert {"kimi_T16384", "gptoss_T4096"} <= set(summ["prefill"])
    assert {"512/4_softmax", "2304/36_softmax"} <= set(summ["router"])
    assert {"deepseek_T1", "deepseek_T4", "deepseek_T16"} <= set(summ["decode"])
