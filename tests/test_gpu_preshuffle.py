"""Weights in fragment order (moe_preshuffle_weights, moe_preshuffle_scales, MOE_PRESHUFFLED).

The layout is a byte permutation, checked against a numpy transposition of the rows.  The
GEMMs read the same operand bytes in the same order either way, so gate-up outputs and
reduce-mode down outputs are bit-identical to the natural layout's, in the decode and the
prefill kernels; moe_forward with preshuffled weights is also held to the oracle's bounds."""

import sys

import numpy as np
import pytest
import torch

import synth
from _gpu_helpers import BF16_COS, BF16_TOL, FP8_TOL, compare_layer, compare_out_bf16_atomic, oracle_route
from test_gpu_layer import oracle_layer, to_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    sys.stderr.write(f"\n[gpu] {request.node.nodeid}\n")
    sys.stderr.flush()
    yield


def fragment_order(raw: np.ndarray) -> np.ndarray:
    """raw uint8 [rows, rowb] -> bytes in the documented order [R][chunk][half][g][i][16]."""
    rows, rowb = raw.shape
    v = raw.reshape(rows // 16, 16, rowb // 128, 2, 4, 16)  # R, i, c, h, g, byte
    return v.transpose(0, 2, 3, 4, 1, 5).reshape(-1)


@pytest.mark.parametrize("dtype,K", [("bf16", 192), ("bf16", 64), ("fp8", 256), ("mxfp4", 512)])
def test_preshuffle_is_the_documented_permutation(dtype, K):
    import mixture_experts_routing_amd as m
    g = torch.Generator().manual_seed(K)
    cols = K // 2 if dtype == "mxfp4" else K
    raw = torch.randint(0, 256, (3, 32, cols * (2 if dtype == "bf16" else 1)), generator=g, dtype=torch.uint8)
    w = raw.view(torch.bfloat16) if dtype == "bf16" else raw
    out = m.moe_preshuffle_weights(dtype, w.cuda())
    torch.cuda.synchronize()
    got = out.cpu().contiguous().view(torch.uint8).numpy().reshape(-1)
    want = fragment_order(raw.numpy().reshape(96, -1))
    assert np.array_equal(got, want)


def scale_fragment_order(raw: np.ndarray) -> np.ndarray:
    """raw uint8 E8M0 scales [rows, K/32] -> bytes in the documented order [R][chunk][i][8]."""
    rows, nsb = raw.shape
    v = raw.reshape(rows // 16, 16, nsb // 8, 8)  # R, i, c, byte
    return v.transpose(0, 2, 1, 3).reshape(-1)


@pytest.mark.parametrize("K", [256, 768, 7168])
def test_preshuffle_scales_is_the_documented_permutation(K):
    import mixture_experts_routing_amd as m
    g = torch.Generator().manual_seed(K)
    raw = torch.randint(0, 256, (3, 32, K // 32), generator=g, dtype=torch.uint8)
    out = m.moe_preshuffle_scales(raw.cuda())
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(-1)
    want = scale_fragment_order(raw.numpy().reshape(96, -1))
    assert np.array_equal(got, want)


def pre_weights(m, dtype, g):
    """w1, w2 in fragment order, and for mxfp4 their E8M0 scales too (fp8 scales unchanged)."""
    out = {"w1": m.moe_preshuffle_weights(dtype, g["w1"]), "w2": m.moe_preshuffle_weights(dtype, g["w2"]),
           "w1_scale": g.get("w1_scale"), "w2_scale": g.get("w2_scale")}
    if dtype == "mxfp4":
        out["w1_scale"] = m.moe_preshuffle_scales(g["w1_scale"])
        out["w2_scale"] = m.moe_preshuffle_scales(g["w2_scale"])
    return out


def _ok(D, I, dtype):
    unit = {"bf16": 64, "fp8": 128, "mxfp4": 256}[dtype]
    return D % unit == 0 and I % unit == 0


SHAPES = [
    # (T, E, k, D, I, B, dtype): decode kernels at BLOCK_M 16/32/64, then the prefill kernels
    (37, 16, 4, 384, 192, 16, "bf16"), (61, 12, 3, 320, 128, 64, "bf16"),
    (300, 8, 2, 320, 192, 64, "bf16"), (640, 8, 4, 384, 512, 64, "bf16"),
    (37, 16, 4, 384, 512, 16, "fp8"), (200, 40, 5, 256, 640, 64, "fp8"),
    (640, 8, 4, 384, 1024, 64, "fp8"), (300, 8, 2, 512, 512, 64, "fp8"),
    (37, 16, 4, 512, 256, 32, "mxfp4"), (300, 8, 2, 512, 256, 64, "mxfp4"),
    (640, 8, 4, 256, 512, 64, "mxfp4"),
]


@pytest.mark.parametrize("T,E,k,D,I,B,dtype", SHAPES)
def test_preshuffled_gemms_bit_identical(T, E, k, D, I, B, dtype):
    import mixture_experts_routing_amd as m
    assert _ok(D, I, dtype)
    g = to_cuda(synth.small_layer_inputs(T, E, k, D, I, dtype, seed=3))
    pw = pre_weights(m, dtype, g)
    r = m.moe_topk_softmax_sort(g["logits"], k, B)
    kw1 = dict(x_scale=g.get("x_scale"), w1_scale=g.get("w1_scale"))
    a0, s0 = m.moe_gemm1_gateup(dtype, g["x"], g["w1"], r, k, B, **kw1)
    a1, s1 = m.moe_gemm1_gateup(dtype, g["x"], pw["w1"], r, k, B, preshuffled=True, x_scale=g.get("x_scale"),
                                w1_scale=pw["w1_scale"])
    torch.cuda.synchronize()
    assert torch.equal(a0, a1)
    if s0 is not None:
        assert torch.equal(s0, s1)
    y0 = m.moe_gemm2_down(dtype, a0, g["w2"], r, T, k, B, "reduce", a_scale=s0, w2_scale=g.get("w2_scale"))
    y1 = m.moe_gemm2_down(dtype, a0, pw["w2"], r, T, k, B, "reduce", preshuffled=True, a_scale=s0,
                          w2_scale=pw["w2_scale"])
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)


FWD = [
    # (T, E, k, D, I, B, dtype, mode): decode and prefill kernels, every output mode; the fp8
    # and mxfp4 shapes have I >= 512, where one requant code one step apart moves an output by
    # about 0.2/sqrt(I) of its rms, well inside the 5e-2 bound
    (37, 16, 4, 384, 192, 16, "bf16", "atomic"), (640, 8, 4, 384, 512, 64, "bf16", "atomic"),
    (200, 40, 5, 256, 640, 64, "fp8", "atomic_bf16"), (640, 8, 4, 384, 1024, 64, "fp8", "reduce"),
    (61, 12, 3, 512, 512, 32, "fp8", "atomic"), (300, 8, 2, 512, 512, 64, "mxfp4", "atomic"),
    (37, 16, 4, 512, 512, 16, "mxfp4", "reduce"), (640, 8, 4, 384, 1024, 64, "fp8", "reduce_bf16"),
    (37, 16, 4, 384, 192, 16, "bf16", "reduce_bf16"),
]


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
@pytest.mark.parametrize("T,E,k,D,I,B,dtype,mode", FWD)
def test_preshuffled_forward_against_oracle(T, E, k, D, I, B, dtype, mode, seed):
    import mixture_experts_routing_amd as m
    cpu = synth.small_layer_inputs(T, E, k, D, I, dtype, seed=1000 * seed + T + D, w_std=0.05)
    g = to_cuda(cpu)
    pw = pre_weights(m, dtype, g)
    out, ws, offs = m.moe_forward(dtype, g["logits"], g["x"], pw["w1"], pw["w2"], k, B, mode,
                                  x_scale=g.get("x_scale"), w1_scale=pw["w1_scale"], w2_scale=pw["w2_scale"],
                                  preshuffled=True)
    torch.cuda.synchronize()
    ref = oracle_layer(cpu, oracle_route(cpu["logits"], k, B), dtype)
    tol = BF16_TOL if dtype == "bf16" else FP8_TOL
    if mode == "atomic_bf16":
        compare_out_bf16_atomic(out, ref, np.arange(T), k, tol)
    else:
        y = m.workspace_views(ws, offs, dtype, mode, T, E, k, D, I, B)["y"]
        compare_layer(out, y, mode, k, ref, np.arange(T), tol, BF16_COS if dtype == "bf16" else None)


def test_preshuffled_deepseek_decode_full_size():
    """The benchmarked DeepSeek-R1 decode shape (T=16): reduce-mode layer output bit-identical
    with preshuffled weights."""
    import mixture_experts_routing_amd as m
    wl = synth.WORKLOADS["deepseek"]
    g = synth.layer_inputs(wl, 16, seed=0, device="cuda")
    w1p = m.moe_preshuffle_weights("bf16", g["w1"])
    w2p = m.moe_preshuffle_weights("bf16", g["w2"])
    o0, _, _ = m.moe_forward("bf16", g["logits"], g["x"], g["w1"], g["w2"], wl.topk, wl.block_m, "reduce")
    o1, _, _ = m.moe_forward("bf16", g["logits"], g["x"], w1p, w2p, wl.topk, wl.block_m, "reduce",
                             preshuffled=True)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1)


@pytest.fixture(scope="module")
def pre_cache():
    cache = {}
    yield cache
    cache.clear()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,T,tokens", [
    ("deepseek", 1, [0]),
    ("deepseek", 2, [0, 1]),
    ("deepseek", 4, [0, 1, 2, 3]),
    ("deepseek", 8, [0, 3, 7]),
    ("deepseek", 16, [0, 9, 15]),
    ("gptoss", 16, [0, 7, 15]),
    ("kimi", 64, [0, 33, 63]),
    ("kimi_mxfp4", 64, [0, 33, 63]),
])
def test_preshuffled_full_size_sampled(name, T, tokens, pre_cache):
    """The decode workloads in the configuration the benchmark times them in: weights in
    fragment order (non-temporal weight loads), the workload's own output mode, moe_forward;
    sampled tokens against the oracle."""
    import mixture_experts_routing_amd as m
    wl = synth.WORKLOADS[name]
    if pre_cache.get("name") != name:
        pre_cache.clear()
        torch.cuda.empty_cache()
        base = synth.layer_inputs(wl, 1, seed=0, device="cuda")
        pre_cache.update(name=name, base=base, pw=pre_weights(m, wl.dtype, base))
    g = dict(pre_cache["base"])
    pw = pre_cache["pw"]
    g["logits"] = synth.logits(T, wl.E, seed=T).cuda()
    g.update({kk: v.cuda() for kk, v in synth.activations(T, wl.D, wl.dtype, seed=T, x_std=wl.x_std).items()})
    out, ws, offs = m.moe_forward(wl.dtype, g["logits"], g["x"], pw["w1"], pw["w2"], wl.topk, wl.block_m,
                                  wl.mode, x_scale=g.get("x_scale"), w1_scale=pw["w1_scale"],
                                  w2_scale=pw["w2_scale"], preshuffled=True)
    torch.cuda.synchronize()
    ref = oracle_layer(g, oracle_route(g["logits"], wl.topk, wl.block_m), wl.dtype, tokens=tokens)
    y = m.workspace_views(ws, offs, wl.dtype, wl.mode, T, wl.E, wl.topk, wl.D, wl.I, wl.block_m)["y"]
    tol, cos = (BF16_TOL, BF16_COS) if wl.dtype == "bf16" else (FP8_TOL, None)
    ratio, c, allow = compare_layer(out, y, wl.mode, wl.topk, ref, np.array(tokens), tol, cos)
    sys.stderr.write(f"[parity] {name} T={T} fragment order: max|err|/rms = {ratio:.4g}, cos {c:.7f}, "
                     f"largest rounding-decision allowance {allow:.3g} rms\n")
