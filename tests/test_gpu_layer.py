"""GPU parity of the two-stage expert GEMM and the whole layer against the oracle.

bf16: max|err| <= 2e-2 * rms(out) and cosine >= 0.9999; fp8: max|err| <= 5e-2 * rms(out).
Small shapes are compared on every output; the full-size workloads on sampled tokens
(the oracle evaluates only the experts those tokens use), in the launch configuration
the benchmark times (moe_forward).
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu_helpers import (ACC_REL, BF16_COS, BF16_TOL, FP8_TOL, PerExpert, check_a_bf16, check_a_fp8, check_a_mx,
                          check_route, compare_layer, compare_out, compare_out_bf16_atomic, compare_slot_rows,
                          host_bits, oracle_route)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    sys.stderr.write(f"\n[gpu] {request.node.nodeid}\n")
    sys.stderr.flush()
    yield


def to_cuda(inp):
    return {key: v.cuda() for key, v in inp.items()}


def oracle_layer(inp, route_ref, dtype, tokens=None, slots=None):
    w1 = PerExpert(inp["w1"])
    w2 = PerExpert(inp["w2"])
    kw = {}
    if dtype in ("fp8", "mxfp4"):
        kw = dict(x_scale=inp["x_scale"].cpu().numpy(), w1_scale=PerExpert(inp["w1_scale"]),
                  w2_scale=PerExpert(inp["w2_scale"]))
    return oracle.moe_layer(host_bits(inp["x"]), w1, w2, route_ref.ids, route_ref.weights, dtype,
                            tokens=tokens, slots=slots, band_rel=ACC_REL[dtype], **kw)


def run_forward(inp, k, B, dtype, mode):
    import mixture_experts_routing_amd as m
    out, ws, offs = m.moe_forward(dtype, inp["logits"], inp["x"], inp["w1"], inp["w2"], k, B, mode,
                                  x_scale=inp.get("x_scale"), w1_scale=inp.get("w1_scale"),
                                  w2_scale=inp.get("w2_scale"))
    torch.cuda.synchronize()
    T = inp["x"].shape[0]
    E, twoI, _ = inp["w1"].shape
    D = inp["w2"].shape[1]  # (x is packed two values per byte in mxfp4)
    views = m.workspace_views(ws, offs, dtype, mode, T, E, k, D, twoI // 2, B)
    return out, views


def check_intermediate(views, ref, dtype, rows):
    """Intermediate a, element by element (after the output checks): the bf16 rows (for fp8 and
    mxfp4 the rows before the requant) inside the oracle's interval, then the fp8 or mxfp4
    scales and dequantised values inside the oracle's ranges."""
    got = views["a" if dtype == "bf16" else "a_pre"].float().cpu().double().numpy()[rows]
    check_a_bf16(got, ref, rows)
    if dtype == "mxfp4":
        check_a_mx(views["a"].cpu().numpy()[rows], views["a_scale"].cpu().numpy()[rows], ref, rows)
    elif dtype == "fp8":
        check_a_fp8(views["a"].cpu().numpy()[rows], views["a_scale"].cpu().numpy()[rows], ref, rows)


SMALL_BF16 = [
    # (T, E, k, D, I, B): tiny workload; shapes spanning several tiles with ragged tails
    (4, 8, 2, 128, 64, 16),
    (37, 16, 4, 384, 192, 16),
    (37, 16, 4, 384, 192, 32),
    (61, 12, 3, 320, 128, 64),
    (5, 6, 6, 192, 256, 32),
    (200, 40, 5, 256, 64, 64),
    # BLOCK_M = 64 with T*k >= 32*E: the LDS-tiled prefill kernels, with a partial channel
    # tile, a partial model_dim tile and a ragged second K stage
    (300, 8, 2, 320, 192, 64),
    (640, 8, 4, 384, 512, 64),
    # long rows (2 KB) through the prefill kernels
    (256, 4, 2, 1024, 1088, 64),
    # decode kernels with K split over the waves of a block (each wave's share of a row is
    # kept at 1 KB or more): gate-up 4 ways (8 KB rows), down 4 ways, both 2 ways (3 KB rows)
    (8, 8, 2, 4096, 64, 16),
    (8, 8, 2, 128, 4096, 32),
    (9, 8, 2, 1536, 1536, 16),
]
# fp8: the intermediate is requantised per row from bf16 values that the GPU (fp32 MFMA
# sums) and the oracle (fp64) may round one bf16 ulp apart; such a pair can land on
# adjacent e4m3 codes.  One flipped code moves an output by about 0.2/sqrt(I) of its
# rms, so the 5e-2 bound is meaningful for I >= 512 (the Kimi shape has I = 512).
SMALL_FP8 = [
    (4, 8, 2, 128, 512, 16),
    (37, 16, 4, 384, 512, 16),
    (37, 16, 4, 320, 576, 32),
    (61, 12, 3, 320, 512, 64),
    (200, 40, 5, 256, 640, 64),
    # prefill kernels; D = 320 and I = 576 leave a half 128-byte chunk at the end of K
    (300, 8, 2, 320, 576, 64),
    (640, 8, 4, 384, 1024, 64),
    # long fp8 rows; 2112-byte rows end in a half 128-byte chunk
    (200, 4, 2, 2112, 2112, 64),
    # decode gate-up with K split 4 ways (8 KB rows)
    (8, 8, 2, 8192, 512, 16),
]
# mxfp4: D and I multiples of 128; every BLOCK_M runs the decode kernels; D = 384 and
# I = 640 end in a half 128-byte chunk (one of the two MFMAs of a chunk)
SMALL_MX = [
    (4, 8, 2, 128, 128, 16),
    (37, 16, 4, 384, 256, 16),
    (37, 16, 4, 256, 640, 32),
    (61, 12, 3, 256, 512, 64),
    (300, 8, 2, 384, 384, 64),
    # BLOCK_M = 64, T*k >= 32*E and D, I multiples of 256: the tiled prefill kernel with its
    # staged block scales (runs of 1-4 blocks, a partial model_dim tile)
    (300, 8, 2, 512, 256, 64),
    (640, 8, 4, 256, 512, 64),
    (256, 4, 2, 1024, 768, 64),
    # decode gate-up with K split 4 ways (4 KB rows of E2M1 codes) and 2 ways (2 KB rows)
    (8, 8, 2, 8192, 256, 16),
    (8, 8, 2, 4096, 256, 32),
]
SMALL = ([(*c, "bf16") for c in SMALL_BF16] + [(*c, "fp8") for c in SMALL_FP8] +
         [(*c, "mxfp4") for c in SMALL_MX])


@pytest.mark.parametrize("mode", ["atomic", "reduce", "reduce_bf16"])
@pytest.mark.parametrize("T,E,k,D,I,B,dtype", SMALL)
def test_layer_small_full_compare(T, E, k, D, I, B, dtype, mode):
    inp = synth.small_layer_inputs(T, E, k, D, I, dtype, seed=T + D, w_std=0.05)
    ref_route = oracle_route(inp["logits"], k, B)
    ref = oracle_layer(inp, ref_route, dtype)
    g = to_cuda(inp)
    out, views = run_forward(g, k, B, dtype, mode)
    check_route({kk: views[kk] for kk in ("topk_weights", "topk_ids", "sorted_token_ids", "expert_ids", "num_valid")},
                ref_route, T, k)
    rows = np.arange(T)
    tol, cos = (BF16_TOL, BF16_COS) if dtype == "bf16" else (FP8_TOL, None)
    compare_layer(out, views["y"], mode, k, ref, rows, tol, cos)
    if mode != "atomic":  # the slot rows themselves
        compare_slot_rows(views["y"], mode, ref, np.arange(T * k), tol, cos)
    check_intermediate(views, ref, dtype, np.arange(T * k))


@pytest.mark.parametrize("T,E,k,D,I,B,dtype", SMALL)
def test_layer_small_atomic_bf16(T, E, k, D, I, B, dtype):
    """Packed bf16 atomic accumulation into out: within the fp32 modes' bound plus the
    allowance of the k + 1 bf16 roundings (decode kernels, the tiled prefill kernel's paired
    epilogue, half chunks)."""
    inp = synth.small_layer_inputs(T, E, k, D, I, dtype, seed=T + D, w_std=0.05)
    ref_route = oracle_route(inp["logits"], k, B)
    ref = oracle_layer(inp, ref_route, dtype)
    out, views = run_forward(to_cuda(inp), k, B, dtype, "atomic_bf16")
    assert views["y"] is None
    compare_out_bf16_atomic(out, ref, np.arange(T), k, BF16_TOL if dtype == "bf16" else FP8_TOL)
    check_intermediate(views, ref, dtype, np.arange(T * k))


@pytest.mark.parametrize("mode", ["atomic", "reduce", "reduce_bf16"])
@pytest.mark.parametrize("dtype,I", [("bf16", 64), ("fp8", 512)])
def test_layer_long_expert_run(dtype, I, mode):
    """One expert holding 65 sorted blocks: prefill tiles of four blocks are counted from the
    expert's first block, which takes the tile-start search past one 64-block step.  With a
    single slot per token and these small random shapes the output has heavy tails (max/rms
    about 7), where one bf16 rounding step of the output alone can exceed 2e-2 * rms; the fp32
    results before that rounding are compared instead (atomic: the accumulator, reduce: the
    slot rows), and the output must be their round-to-nearest-even bf16 value."""
    T, E, k, D, B = 4160, 1, 1, 128, 64
    inp = synth.small_layer_inputs(T, E, k, D, I, dtype, seed=T + D, w_std=0.05)
    ref_route = oracle_route(inp["logits"], k, B)
    ref = oracle_layer(inp, ref_route, dtype)
    out, views = run_forward(to_cuda(inp), k, B, dtype, mode)
    y = views["y"]
    tol = BF16_TOL if dtype == "bf16" else FP8_TOL
    if mode == "atomic":
        compare_out(y, ref.out, np.arange(T), tol, BF16_COS, allow=ref.out_allow)
    else:
        compare_slot_rows(y, mode, ref, np.arange(T * k), tol, BF16_COS)
    fin = y if mode == "atomic" else y.view(T, k, D).float().sum(1)
    assert torch.equal(out, fin.to(torch.bfloat16))


def test_layer_staged_calls_match_forward():
    """The four calls chained by hand give the same output as moe_forward."""
    import mixture_experts_routing_amd as m
    T, E, k, D, I, B = 33, 10, 3, 256, 128, 32
    for dtype in ("bf16", "fp8"):
        g = to_cuda(synth.small_layer_inputs(T, E, k, D, I, dtype, seed=1))
        r = m.moe_topk_softmax_sort(g["logits"], k, B)
        a, a_scale = m.moe_gemm1_gateup(dtype, g["x"], g["w1"], r, k, B, x_scale=g.get("x_scale"),
                                        w1_scale=g.get("w1_scale"))
        y = m.moe_gemm2_down(dtype, a, g["w2"], r, T, k, B, "reduce", a_scale=a_scale,
                             w2_scale=g.get("w2_scale"))
        out = m.moe_finalize("reduce", y, T, k, D)
        out_f, _ = run_forward(g, k, B, dtype, "reduce")
        torch.cuda.synchronize()
        assert torch.equal(out, out_f)  # same kernels, same order: bit-identical


def test_layer_empty_tokens():
    import mixture_experts_routing_amd as m
    g = to_cuda(synth.small_layer_inputs(1, 8, 2, 128, 64, "bf16"))
    x = g["x"][:0]
    out, _, _ = m.moe_forward("bf16", g["logits"][:0], x, g["w1"], g["w2"], 2, 16, "atomic",
                              workspace=torch.empty(1024, dtype=torch.uint8, device="cuda"))
    assert out.shape == (0, 128)


def test_layer_distinct_slot_weights_catch_slot0_gather():
    """Two picks per token with very different weights and experts: a gather that
    reads slot 0 for every slot would be far outside tolerance."""
    T, E, k, D, I, B = 16, 8, 2, 128, 64, 16
    inp = synth.small_layer_inputs(T, E, k, D, I, "bf16", seed=21, w_std=0.1)
    inp["logits"][:, 0] += 1.5  # expert 0 is usually first with a large weight
    ref_route = oracle_route(inp["logits"], k, B)
    ref = oracle_layer(inp, ref_route, "bf16")
    out, views = run_forward(to_cuda(inp), k, B, "bf16", "atomic")
    compare_layer(out, views["y"], "atomic", k, ref, np.arange(T), BF16_TOL, BF16_COS)


# ----------------------------------------------------------------------------- full-size workloads
def spread(T, n=32):
    """n token indices spread evenly over [0, T), first and last included."""
    return sorted(set(np.linspace(0, T - 1, n).round().astype(int).tolist()))


FULL = [
    # (workload, T, sampled tokens): every DeepSeek-R1 decode size, the GPT-OSS and Kimi-K2.5
    # decode sizes, and 32 tokens spread over each prefill size
    ("deepseek", 1, [0]),
    ("deepseek", 2, [0, 1]),
    ("deepseek", 4, [0, 1, 2, 3]),
    ("deepseek", 8, list(range(8))),
    ("deepseek", 16, [0, 5, 9, 15]),
    ("gptoss", 16, [0, 7, 15]),
    ("gptoss", 4096, spread(4096)),
    ("kimi", 64, list(range(0, 64, 4)) + [63]),
    ("kimi", 4096, spread(4096)),
    ("kimi", 16384, spread(16384)),
    # the largest T the layer calls accept at this shape (T*k*D < 2^31): the prefill GEMMs at
    # their largest gathered-row offsets
    ("kimi", 33288, spread(33288)),
    ("kimi_mxfp4", 64, list(range(0, 64, 4)) + [63]),
    ("kimi_mxfp4", 4096, spread(4096)),
    ("kimi_mxfp4", 16384, spread(16384)),
]


@pytest.fixture(scope="module")
def weights_cache():
    cache = {}
    yield cache
    cache.clear()
    torch.cuda.empty_cache()


def report(name, T, what, res):
    ratio, cos, allow = res
    sys.stderr.write(f"[parity] {name} T={T} {what}: max|err|/rms = {ratio:.4g}, cos {cos:.7f}, "
                     f"largest rounding-decision allowance {allow:.3g} rms\n")
    sys.stderr.flush()


def largest_tile_slots(views, B):
    """Slot rows of the first prefill tile of the expert with the most blocks: up to four
    consecutive blocks counted from the expert's first block (all real slots when the expert
    has more blocks than the tile)."""
    eid = views["expert_ids"].cpu().numpy()
    nv = int(views["num_valid"].item())
    blocks = eid[: nv // B]
    experts, first, count = np.unique(blocks, return_index=True, return_counts=True)
    e = int(np.argmax(count))
    b0, nb = int(first[e]), min(4, int(count[e]))
    sid = views["sorted_token_ids"].cpu().numpy()[b0 * B:(b0 + nb) * B]
    return sid, nb, int(count[e])


@pytest.mark.parametrize("name,T,tokens", FULL)
def test_layer_full_size_sampled(name, T, tokens, weights_cache):
    wl = synth.WORKLOADS[name]
    if weights_cache.get("name") != name:
        weights_cache.clear()
        torch.cuda.empty_cache()
        base = synth.layer_inputs(wl, 1, seed=0, device="cuda")
        weights_cache.update(name=name, base=base)
    # token-dependent inputs for this T; the weights are shared by the T values of a workload
    inp = dict(weights_cache["base"])
    inp["logits"] = synth.logits(T, wl.E, seed=T).cuda()
    inp.update({key: v.cuda() for key, v in synth.activations(T, wl.D, wl.dtype, seed=T, x_std=wl.x_std).items()})
    ref_route = oracle_route(inp["logits"], wl.topk, wl.block_m)
    out, views = run_forward(inp, wl.topk, wl.block_m, wl.dtype, wl.mode)
    check_route({kk: views[kk] for kk in ("topk_weights", "topk_ids", "sorted_token_ids", "expert_ids", "num_valid")},
                ref_route, T, wl.topk)
    tile = None
    if T >= 4096:
        # every slot row of one whole prefill tile, in both reduce modes (the slot rows themselves)
        sid, nb, nblocks = largest_tile_slots(views, wl.block_m)
        tile = sid[sid < T * wl.topk]
    ref = oracle_layer(inp, ref_route, wl.dtype, tokens=tokens, slots=tile)
    rows = np.array(tokens)
    tol, cos = (BF16_TOL, BF16_COS) if wl.dtype == "bf16" else (FP8_TOL, None)
    res = compare_layer(out, views["y"], wl.mode, wl.topk, ref, rows, tol, cos)
    report(name, T, f"{len(rows)} tokens, {wl.mode}", res)
    slots = np.concatenate([np.arange(t * wl.topk, (t + 1) * wl.topk) for t in tokens])
    check_intermediate(views, ref, wl.dtype, slots)
    if tile is not None:
        for mode in ("reduce", "reduce_bf16"):
            if mode == wl.mode:
                out_r, y_r = out, views["y"]
            else:
                out_r, v_r = run_forward(inp, wl.topk, wl.block_m, wl.dtype, mode)
                y_r = v_r["y"]
                res = compare_layer(out_r, y_r, mode, wl.topk, ref, rows, tol, cos)
                report(name, T, f"{len(rows)} tokens, {mode}", res)
            res = compare_slot_rows(y_r, mode, ref, tile, tol, cos)
            report(name, T, f"{mode} slot rows of a {nb}-block tile ({len(tile)} rows; the expert has {nblocks} blocks)",
                   res)
            del out_r, y_r
            torch.cuda.empty_cache()
    if name in ("deepseek", "kimi") and T in (16, 16384):
        # the same inputs with packed bf16 atomics into out
        out2, _ = run_forward(inp, wl.topk, wl.block_m, wl.dtype, "atomic_bf16")
        used = compare_out_bf16_atomic(out2, ref, rows, wl.topk, tol)
        sys.stderr.write(f"[parity] {name} T={T} packed bf16 atomics: {used:.3g} of the allowance used\n")


@pytest.mark.parametrize("skew", [False, True])
@pytest.mark.parametrize("mode", ["reduce", "atomic"])
def test_layer_short_rows_no_k_split(mode, skew):
    """Decode down projection with BLOCK_M 64, no K split (n_act * D/32 >= 256*16*12 waves) and
    rows of at most 1 KB (bf16 I = 256): the kernel variant with four 16-row weight groups per
    wave.  Its blocks with at most 16 real rows run the first row group alone; with skew, two
    experts that every token prefers fill whole 64-row blocks, so both forms run in one launch.
    Sampled tokens against the oracle."""
    T, E, k, D, I, B = 64, 256, 8, 7168, 256, 64
    wl = synth.Workload("short_rows", E, k, D, I, B, "bf16", mode, 1.0, 0.02)
    inp = synth.layer_inputs(wl, T, seed=11, device="cuda")
    if skew:
        inp["logits"][:, :2] += 6.0
    ref_route = oracle_route(inp["logits"], k, B)
    # the library sizes the K split from min(T*k, E) experts (before routing is known)
    assert min(T * k, E) * (D // 32) >= 256 * 16 * 12 and 2 * I <= 1024 and T * k < 32 * E
    out, views = run_forward(inp, k, B, "bf16", mode)
    tokens = [0, 31, 63]
    ref = oracle_layer(inp, ref_route, "bf16", tokens=tokens)
    compare_layer(out, views["y"], mode, k, ref, np.array(tokens), BF16_TOL, BF16_COS)
    del inp
    torch.cuda.empty_cache()
