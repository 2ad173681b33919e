"""moe_forward_noalloc (the workspace in the library's static per-device array) against
moe_forward with a caller workspace: the same kernels in the same order.  Reduce mode is
deterministic, so the outputs must be bit-identical; fp32 atomic adds land in any order, so
atomic mode must agree within one bf16 step and the layer bound.  Each case makes two calls
in a row, the second with fewer tokens, so the array's leftovers from the first call must not
leak into the second."""

import sys

import numpy as np
import pytest
import torch

import synth
from _gpu_helpers import BF16_TOL, bf16_ulp, compare_out, compare_out_bf16_atomic, oracle_route
from test_gpu_layer import oracle_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    sys.stderr.write(f"\n[gpu] {request.node.nodeid}\n")
    sys.stderr.flush()
    yield


CASES = [
    # (E, k, D, I, B, dtype, mode, T first, T second)
    (64, 8, 1024, 512, 16, "bf16", "atomic", 16, 5),
    (64, 8, 1024, 512, 16, "bf16", "reduce", 16, 5),
    (32, 4, 512, 512, 64, "fp8", "reduce", 96, 3),
    (32, 4, 512, 512, 64, "fp8", "atomic", 96, 3),
    (32, 4, 512, 512, 64, "fp8", "reduce_bf16", 96, 3),
    (16, 2, 512, 256, 32, "mxfp4", "reduce", 40, 7),
    (16, 4, 256, 128, 16, "bf16", "atomic_bf16", 12, 2),
]


@pytest.mark.parametrize("E,k,D,I,B,dtype,mode,T1,T2", CASES)
def test_noalloc_matches_forward(E, k, D, I, B, dtype, mode, T1, T2):
    import mixture_experts_routing_amd as m
    assert m.moe_forward_workspace_bytes(dtype, mode, T1, E, k, D, I, B) <= m.moe_forward_noalloc_max_bytes()
    w = {kk: v.cuda() for kk, v in synth.small_layer_inputs(1, E, k, D, I, dtype, seed=E + D).items()}
    for T in (T1, T2):
        tok = {"logits": synth.logits(T, E, seed=T).cuda()}
        tok.update({kk: v.cuda() for kk, v in synth.activations(T, D, dtype, seed=T).items()})
        kw = dict(x_scale=tok.get("x_scale"), w1_scale=w.get("w1_scale"), w2_scale=w.get("w2_scale"))
        ref, _, _ = m.moe_forward(dtype, tok["logits"], tok["x"], w["w1"], w["w2"], k, B, mode, **kw)
        out = torch.full((T, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        m.moe_forward_noalloc(dtype, tok["logits"], tok["x"], w["w1"], w["w2"], k, B, out, mode, **kw)
        torch.cuda.synchronize()
        if mode in ("reduce", "reduce_bf16"):
            assert torch.equal(out, ref), f"T={T}: {mode} outputs differ"
        elif mode == "atomic":
            # the same fp32 adds in another order (a few fp32 roundings), then one bf16 rounding
            a = out.float().cpu().double().numpy()
            b = ref.float().cpu().double().numpy()
            assert np.isfinite(a).all()
            rms = float(np.sqrt(np.mean(b * b)))
            assert np.all(np.abs(a - b) <= bf16_ulp(np.maximum(np.abs(a), np.abs(b))) + 2.0 ** -20 * rms), \
                f"T={T}: atomic-mode outputs differ by more than one bf16 step"
            compare_out(out, b, np.arange(T), BF16_TOL, None)
        else:
            # packed bf16 atomics: both results within that mode's allowance of the oracle
            cpu = {kk: v.cpu() for kk, v in {**w, **tok}.items()}
            r = oracle_route(cpu["logits"], k, B)
            o = oracle_layer(cpu, r, dtype)
            for got in (out, ref):
                compare_out_bf16_atomic(got, o, np.arange(T), k, BF16_TOL)
        sys.stderr.write(f"[noalloc] {dtype} {mode} T={T}: matches moe_forward\n")
