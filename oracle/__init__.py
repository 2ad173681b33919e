"""CPU oracle for the MoE-layer forward hot path (routing + two-stage expert GEMM).

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain, obviously-correct
definition that the HIP path is checked against.  Only the test suite, the
smoke check and the CPU-baseline leg of the benchmark may import it; the
product path (the C-ABI library and its Python binding) never does, and the
two share no code.

Arithmetic is float64 unless a step's decision is an integer taken from a
floating-point value (a quantised code), in which case the step states the
precision it uses.  Every function cites the passage of the source pages it
follows:

* "[Feat] Fuse TopKGatingSoftmax and MoE Sorting kernels" (ROCm/FlyDSL #582)
  -- routing: top-k gating softmax fused with MoE sorting.
* "[MoE] Port moe_gemm_2stage (stage1+stage2) to the new fx.* pipeline -- fp8"
  (ROCm/FlyDSL #947) -- the two-stage expert GEMM and its epilogue modes.
* "[Common] Optimize fused router forward/backward kernels"
  (NVIDIA/TransformerEngine #3012) -- score functions and the host checks.
* "[RadeonFlow] flydsl mxfp4 a4w4 MoE: bring gemm1/gemm2 to parity with the
  HIP backend" (ROCm/aiter #3828) -- the Kimi-K2.5 shape and the mxfp4 (a4w4) GEMMs.

Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle_*.py`` (brute force, closed forms, invariants, library
special cases, codec tables).  The pages print no output value for any
layer, so absolute layer outputs are pinned only through those checks.
"""

from .codecs import (
    bf16_decode,
    bf16_encode_rne,
    e2m1_decode,
    e2m1_encode_rne_sat,
    e4m3_decode,
    e4m3_encode_rne_sat,
    e8m0_decode,
    fp4_pack,
    fp4_unpack,
    mx_dequantize,
    mx_quantize,
    E2M1_MAX,
    E2M1_TABLE,
    E4M3_MAX,
    MX_BLOCK,
)
from .routing import (
    RouteResult,
    aux_loss_scores,
    aux_loss_scores_backward,
    aux_loss_scores_f64,
    group_scores,
    route,
    route_grouped,
    routing_weights,
    routing_weights_backward,
    routing_weights_f64,
    select_groups,
    select_topk,
    select_topk_grouped,
    sort_slots,
    sorted_capacity,
)
from .layer import LayerResult, moe_layer

__all__ = [
    "bf16_decode",
    "bf16_encode_rne",
    "e2m1_decode",
    "e2m1_encode_rne_sat",
    "e4m3_decode",
    "e4m3_encode_rne_sat",
    "e8m0_decode",
    "fp4_pack",
    "fp4_unpack",
    "mx_dequantize",
    "mx_quantize",
    "E2M1_MAX",
    "E2M1_TABLE",
    "E4M3_MAX",
    "MX_BLOCK",
    "RouteResult",
    "aux_loss_scores",
    "aux_loss_scores_backward",
    "aux_loss_scores_f64",
    "group_scores",
    "route",
    "route_grouped",
    "routing_weights",
    "routing_weights_backward",
    "routing_weights_f64",
    "select_groups",
    "select_topk",
    "select_topk_grouped",
    "sort_slots",
    "sorted_capacity",
    "LayerResult",
    "moe_layer",
]
