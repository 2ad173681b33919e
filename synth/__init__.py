"""Seeded synthetic inputs for the MoE-layer workloads.

This module only draws random tensors and packs them into the storage
formats the path consumes.  It holds none of the layer's arithmetic and is
shared by the tests, the benchmark and the smoke check; both the CPU oracle
and the HIP path receive exactly the tensors produced here.

Workloads (shapes from the statement of the problem and the pages' model
shapes: DeepSeek-R1 and GPT-OSS-120B on the fused-routing page, the
E/topk sweep of the TransformerEngine router page, Kimi-K2.5's TP=4 expert
share on the aiter mxfp4 page):

* tiny:     T=4, E=8, topk=2, D=128, I=64, BLOCK_M=16, bf16
* deepseek: T in {1,2,4,8,16}, E=256, topk=8, D=7168, I=2048, BLOCK_M=16, bf16, atomic
* gptoss:   E=128, topk=4, D=I=2880, T=16 (decode) / 4096 (prefill), BLOCK_M=64, bf16, reduce
* router:   T=8192, E/topk in {512/4, 512/22, 2304/36}, softmax|sigmoid, BLOCK_M=32
* router_grouped: E=256, topk=8 in 8 groups of 32, 4 groups kept (the DeepSeek-V3 routing
            shape), sigmoid, T=16 (BLOCK_M=16) and T=8192 (BLOCK_M=32)
* aux scores: T=8192, E/topk in {512/22, 2304/36}, softmax|sigmoid
* kimi:     E=385, topk=9, D=7168, I=512, T in {64, 4096, 16384}, BLOCK_M=64, fp8, atomic
* kimi_mxfp4: the kimi shape with mxfp4 (a4w4) activations and weights

Distributions: router logits fp32 N(0,1); activations N(0,1) (gptoss:
N(0,0.02)); weights N(0,0.02).  fp8 inputs: activations get one scale per
token and weights one scale per output channel, scale = amax / 448, values
cast with torch's e4m3fn conversion of value/scale.  mxfp4 inputs are drawn
directly in their storage format, so no quantisation happens here: every byte
of the packed E2M1 codes is uniform (two uniform codes), and each block of 32
elements along K gets an E8M0 exponent uniform in 125..127 for activations
(rms about 0.7) and 119..121 for weights (rms about 0.02).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import torch

FP8_MAX = 448.0


@dataclass(frozen=True)
class Workload:
    name: str
    E: int
    topk: int
    D: int
    I: int
    block_m: int
    dtype: str          # "bf16" | "fp8" | "mxfp4"
    mode: str           # "atomic" | "reduce"
    x_std: float
    w_std: float
    tokens: tuple = field(default_factory=tuple)


WORKLOADS = {
    "tiny": Workload("tiny", 8, 2, 128, 64, 16, "bf16", "atomic", 1.0, 0.02, (4,)),
    "deepseek": Workload("deepseek", 256, 8, 7168, 2048, 16, "bf16", "atomic", 1.0, 0.02,
                         (1, 2, 4, 8, 16)),
    "gptoss": Workload("gptoss", 128, 4, 2880, 2880, 64, "bf16", "reduce", 0.02, 0.02,
                       (16, 4096)),
    "kimi": Workload("kimi", 385, 9, 7168, 512, 64, "fp8", "atomic", 1.0, 0.02,
                     (64, 4096, 16384)),
    "kimi_mxfp4": Workload("kimi_mxfp4", 385, 9, 7168, 512, 64, "mxfp4", "atomic", 1.0, 0.02,
                           (64, 4096, 16384)),
}

# E8M0 exponent ranges of the random mxfp4 blocks
MX_X_EXP = (125, 127)
MX_W_EXP = (119, 121)

# router-only stress cases: (E, topk); T = 8192, BLOCK_M = 32
ROUTER_T = 8192
ROUTER_BLOCK_M = 32
ROUTER_CASES = ((512, 4), (512, 22), (2304, 36))
# Auxiliary-loss score shapes (E, topk): the two configurations with aux_loss rows in the
# fused-router benchmark tables.
AUX_CASES = ((512, 22), (2304, 36))


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def logits(T: int, E: int, seed: int = 0) -> torch.Tensor:
    """Router logits fp32 [T, E] ~ N(0,1), drawn on the CPU."""
    return torch.randn(T, E, generator=_gen(seed, "cpu"), dtype=torch.float32)


def _quant_rows_e4m3(v: torch.Tensor):
    """fp32 rows -> (uint8 e4m3fn codes, fp32 per-row scale); input preparation only."""
    amax = v.abs().amax(dim=-1).to(torch.float32)
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    codes = (v / scale.unsqueeze(-1)).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return codes.view(torch.uint8), scale


def _mx_random(rows: tuple, n: int, exps: tuple, gen: torch.Generator, device):
    """Random mxfp4 storage: packed codes uint8 [*rows, n/2] and E8M0 exponents uint8
    [*rows, n/32] uniform in exps (inclusive)."""
    packed = torch.randint(0, 256, (*rows, n // 2), generator=gen, dtype=torch.uint8, device=device)
    scale = torch.randint(exps[0], exps[1] + 1, (*rows, n // 32), generator=gen, dtype=torch.uint8, device=device)
    return packed, scale


def activations(T: int, D: int, dtype: str, seed: int = 0, x_std: float = 1.0) -> dict:
    """Token activations on the CPU: {"x": bf16 [T,D]}, {"x": uint8 e4m3 [T,D], "x_scale": fp32 [T]}
    or mxfp4 {"x": packed uint8 [T, D/2], "x_scale": uint8 E8M0 [T, D/32]}."""
    if dtype == "mxfp4":
        xp, xs = _mx_random((T,), D, MX_X_EXP, _gen(seed + 2, "cpu"), "cpu")
        return {"x": xp, "x_scale": xs}
    x32 = torch.randn(T, D, generator=_gen(seed + 2, "cpu"), dtype=torch.float32) * x_std
    if dtype == "bf16":
        return {"x": x32.to(torch.bfloat16)}
    xc, xs = _quant_rows_e4m3(x32)
    return {"x": xc, "x_scale": xs}


def layer_inputs(wl: Workload, T: int, seed: int = 0, device="cpu") -> dict:
    """All inputs of one layer call; weights are drawn per expert on `device`.

    Returns a dict with logits fp32 [T,E] (on `device`), x ([T,D] bf16, or
    uint8 e4m3 codes + x_scale fp32 [T]), w1 [E,2I,D], w2 [E,D,I] (bf16, or
    uint8 codes + w1_scale [E,2I] / w2_scale [E,D]).  mxfp4: x packed [T, D/2] +
    x_scale [T, D/32], w1 [E, 2I, D/2] + w1_scale [E, 2I, D/32], w2 [E, D, I/2] +
    w2_scale [E, D, I/32] (uint8 throughout).
    """
    E, D, I = wl.E, wl.D, wl.I
    lg = logits(T, E, seed)
    if wl.dtype == "mxfp4":
        out = {"logits": lg.to(device)}
        xp, xs = _mx_random((T,), D, MX_X_EXP, _gen(seed + 2, "cpu"), "cpu")
        out["x"], out["x_scale"] = xp.to(device), xs.to(device)
        gw = _gen(seed + 1, device)
        w1 = torch.empty(E, 2 * I, D // 2, dtype=torch.uint8, device=device)
        w2 = torch.empty(E, D, I // 2, dtype=torch.uint8, device=device)
        w1s = torch.empty(E, 2 * I, D // 32, dtype=torch.uint8, device=device)
        w2s = torch.empty(E, D, I // 32, dtype=torch.uint8, device=device)
        for e in range(E):
            w1[e], w1s[e] = _mx_random((2 * I,), D, MX_W_EXP, gw, device)
            w2[e], w2s[e] = _mx_random((D,), I, MX_W_EXP, gw, device)
        out.update(w1=w1, w2=w2, w1_scale=w1s, w2_scale=w2s)
        return out
    gx = _gen(seed + 2, "cpu")
    x32 = torch.randn(T, D, generator=gx, dtype=torch.float32) * wl.x_std
    gw = _gen(seed + 1, device)
    out = {"logits": lg.to(device)}
    if wl.dtype == "bf16":
        out["x"] = x32.to(torch.bfloat16).to(device)
        w1 = torch.empty(E, 2 * I, D, dtype=torch.bfloat16, device=device)
        w2 = torch.empty(E, D, I, dtype=torch.bfloat16, device=device)
        for e in range(E):
            w1[e] = (torch.randn(2 * I, D, generator=gw, device=device) * wl.w_std).to(torch.bfloat16)
            w2[e] = (torch.randn(D, I, generator=gw, device=device) * wl.w_std).to(torch.bfloat16)
        out["w1"], out["w2"] = w1, w2
    else:
        xc, xs = _quant_rows_e4m3(x32)
        out["x"], out["x_scale"] = xc.to(device), xs.to(device)
        w1 = torch.empty(E, 2 * I, D, dtype=torch.uint8, device=device)
        w2 = torch.empty(E, D, I, dtype=torch.uint8, device=device)
        w1s = torch.empty(E, 2 * I, dtype=torch.float32, device=device)
        w2s = torch.empty(E, D, dtype=torch.float32, device=device)
        for e in range(E):
            c, s = _quant_rows_e4m3(torch.randn(2 * I, D, generator=gw, device=device) * wl.w_std)
            w1[e], w1s[e] = c, s
            c, s = _quant_rows_e4m3(torch.randn(D, I, generator=gw, device=device) * wl.w_std)
            w2[e], w2s[e] = c, s
        out.update(w1=w1, w2=w2, w1_scale=w1s, w2_scale=w2s)
    return out


def small_layer_inputs(T: int, E: int, topk: int, D: int, I: int, dtype: str = "bf16",
                       seed: int = 0, x_std: float = 1.0, w_std: float = 0.02) -> dict:
    """CPU inputs for an arbitrary small shape (parity and edge cases)."""
    wl = Workload("custom", E, topk, D, I, 16, dtype, "atomic", x_std, w_std)
    return layer_inputs(wl, T, seed, "cpu")
