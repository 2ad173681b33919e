"""moe_forward captured in a HIP graph: every replay matches the eager call.

Replays are separated by unrelated eager work and synchronisations.  Reduce mode is
deterministic (bit-identical); atomic mode adds the k slots of a token in arbitrary order,
so its bf16 output may move by one ulp; packed bf16 atomics round after every add, so
their output may move by up to (k + 1) half-steps of bf16 at the row's magnitude.
"""

import sys

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    sys.stderr.write(f"\n[gpu] {request.node.nodeid}\n")
    sys.stderr.flush()
    yield


CASES = [
    # (T, E, k, D, I, B, dtype, mode): single-workgroup routing; multi-workgroup routing;
    # the tiled prefill GEMMs; fp8 with the row requant
    (4, 8, 2, 128, 64, 16, "bf16", "atomic"),
    (100, 1100, 4, 128, 64, 16, "bf16", "reduce"),
    (300, 8, 2, 320, 192, 64, "bf16", "reduce"),
    (300, 8, 2, 320, 576, 64, "fp8", "atomic"),
    (300, 8, 2, 320, 192, 64, "bf16", "atomic_bf16"),
    (37, 16, 4, 384, 192, 16, "bf16", "atomic_bf16"),
    (37, 16, 4, 384, 256, 16, "mxfp4", "atomic"),
    (300, 8, 2, 320, 576, 64, "fp8", "reduce_bf16"),
    (37, 16, 4, 384, 192, 16, "bf16", "reduce_bf16"),
]


@pytest.mark.parametrize("T,E,k,D,I,B,dtype,mode", CASES)
def test_forward_graph_replays_match_eager(T, E, k, D, I, B, dtype, mode):
    import mixture_experts_routing_amd as m
    g_in = {key: v.cuda() for key, v in synth.small_layer_inputs(T, E, k, D, I, dtype, seed=T).items()}
    total, _ = m.moe_forward_workspace_layout(dtype, mode, T, E, k, D, I, B)
    ws = torch.empty(total, dtype=torch.uint8, device="cuda")
    out = torch.empty(T, D, dtype=torch.bfloat16, device="cuda")

    def call(stream):
        m.moe_forward(dtype, g_in["logits"], g_in["x"], g_in["w1"], g_in["w2"], k, B, mode,
                      x_scale=g_in.get("x_scale"), w1_scale=g_in.get("w1_scale"),
                      w2_scale=g_in.get("w2_scale"), workspace=ws, out=out, stream=stream)

    call(torch.cuda.current_stream())
    torch.cuda.synchronize()
    eager = out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(torch.cuda.current_stream())
    for rep in range(3):
        out.fill_(float("nan"))
        junk = torch.randn(4096, device="cuda").cumsum(0)  # unrelated eager work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(out.float()).all(), f"replay {rep}"
        if mode in ("reduce", "reduce_bf16"):
            assert torch.equal(out, eager), f"replay {rep} differs from the eager call"
        elif mode == "atomic_bf16":
            diff = (out.float() - eager.float()).abs()
            lim = (k + 1) * 2.0 ** -8 * eager.float().abs().amax(dim=1, keepdim=True)
            assert (diff <= lim).all(), f"replay {rep}: max diff {diff.max().item()}"
        else:
            diff = (out.float() - eager.float()).abs()
            ulp = eager.float().abs().clamp_min(2.0 ** -100) * 2.0 ** -7
            assert (diff <= ulp).all(), f"replay {rep}: max diff {diff.max().item()}"
        del junk
