"""The MoE layer: gate-up GEMM with SiLU-mul, down GEMM, routed weight, combine.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "[MoE] Port moe_gemm_2stage (stage1+stage2) to the new fx.* pipeline
-- fp8 (gfx942 + gfx950)" (ROCm/FlyDSL #947):
* the gate-up helper commit: stage 1 computes silu(gate) * up with optional
  fp8 weight/activation dequant, producing bf16;
* the stage-2 commit: the down projection dequantises per token (row) and
  per output channel (model_dim), optionally multiplies by the routed
  weight, and either atomically adds into out[token, model_dim] or stores
  out[token*topk + slot, model_dim] for a separate reduction;
* padding (sentinel) rows contribute zero.
The workload statement fixes the tensor shapes: router logits [T, E],
gate-up weights [E, 2I, D], down weights [E, D, I], out [T, D].

Readings (listed with the design notes):
* rows [0, I) of each expert's gate-up matrix are the gate, rows [I, 2I) the up;
* silu(z) = z / (1 + exp(-z)); the intermediate a = bf16(silu(g) * u) is
  rounded once (round-to-nearest-even);
* fp8: x is e4m3 with one fp32 scale per token, weights are e4m3 with one
  fp32 scale per output channel; the intermediate is requantised per slot
  row: scale = fp32(amax / 448) (1.0 if the row is all zero), code =
  e4m3_rne_sat(fp32(a / scale)).  This decision is taken in fp32, the
  precision of the kernel that makes it;
* mxfp4 ("[RadeonFlow] flydsl mxfp4 a4w4 MoE", ROCm/aiter #3828: 4-bit activations
  and weights in both GEMMs): x, W1 and W2 are MX blocks (E2M1 codes, one E8M0 scale
  per 32 consecutive elements along K; formats in codecs.py); the bf16 intermediate is
  requantised to MX blocks of 32 along I before the down GEMM.  The block exponent and
  codes are exact functions of the bf16 values, so no precision choice enters;
* the routed weight multiplies the down-projection output before the
  combine; the combined output is kept in float64, unrounded.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .codecs import (bf16_decode, bf16_encode_rne, e4m3_decode, e4m3_encode_rne_sat, E4M3_MAX,
                     fp4_unpack, mx_dequantize, mx_quantize)


def _silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def requant_rows_fp8(a_bits: np.ndarray):
    """Per-row e4m3 requantisation of bf16 rows; returns (codes uint8, scale fp32, dequantised fp64)."""
    a32 = (a_bits.astype(np.uint32) << np.uint32(16)).view(np.float32)  # exact bf16 -> fp32
    amax = np.abs(a32).max(axis=1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    v = (a32 / scale[:, None]).astype(np.float32)  # fp32 division, correctly rounded
    codes = e4m3_encode_rne_sat(v.astype(np.float64))
    deq = e4m3_decode(codes) * scale[:, None].astype(np.float64)
    return codes, scale, deq


def requant_rows_mx(a_bits: np.ndarray):
    """MX requantisation of bf16 rows in blocks of 32; returns (codes uint8 [n, I], scale
    codes uint8 [n, I/32], dequantised fp64)."""
    codes, sc = mx_quantize(bf16_decode(a_bits))
    return codes, sc, mx_dequantize(codes, sc)


@dataclass
class LayerResult:
    out: np.ndarray       # float64 [T, D]; rows not requested are NaN
    contrib: np.ndarray   # float64 [T*k, D]: routed-weighted down output of each slot
    a_bits: np.ndarray    # uint16 [T*k, I]: bf16 intermediate silu(g)*u (pre-requant)
    a_codes: np.ndarray | None   # uint8 [T*k, I]: fp8 codes, or mxfp4 codes (one per byte)
    a_scale: np.ndarray | None   # float32 [T*k] (fp8), or uint8 E8M0 [T*k, I/32] (mxfp4)
    computed: np.ndarray  # bool [T*k]: slots that were evaluated


def moe_layer(x, w1, w2, ids, weights, dtype: str = "bf16", x_scale=None,
              w1_scale=None, w2_scale=None, tokens=None) -> LayerResult:
    """Reference forward of one MoE layer.

    x: bf16 bits uint16 [T, D] (fp8: e4m3 codes uint8 [T, D] with x_scale fp32 [T];
       mxfp4: packed uint8 [T, D/2] with x_scale uint8 E8M0 [T, D/32]).
    w1: per-expert indexable, w1[e] is [2I, D] (bf16 bits or e4m3 codes with
        w1_scale[e] fp32 [2I]; mxfp4: packed [2I, D/2] with scales [2I, D/32]);
        w2[e] is [D, I] (with w2_scale[e] fp32 [D]; mxfp4: [D, I/2], [D, I/32]).
    ids int32 [T, k], weights fp32 [T, k] from routing.
    tokens: optional iterable of token indices to evaluate (others are NaN);
        only the experts those tokens use are read.
    """
    if dtype not in ("bf16", "fp8", "mxfp4"):
        raise ValueError("dtype must be 'bf16', 'fp8' or 'mxfp4'")
    ids = np.asarray(ids, dtype=np.int64)
    weights = np.asarray(weights, dtype=np.float32)
    T, k = ids.shape
    D = np.asarray(x).shape[1] * (2 if dtype == "mxfp4" else 1)
    tok_mask = np.zeros(T, dtype=bool)
    if tokens is None:
        tok_mask[:] = True
    else:
        tok_mask[np.asarray(list(tokens), dtype=np.int64)] = True

    def dec_x(rows):
        if dtype == "bf16":
            return bf16_decode(np.asarray(x)[rows])
        if dtype == "mxfp4":
            return mx_dequantize(fp4_unpack(np.asarray(x)[rows]), np.asarray(x_scale)[rows])
        return e4m3_decode(np.asarray(x)[rows]) * np.asarray(x_scale, dtype=np.float32)[rows, None].astype(np.float64)

    def dec_w(w, scale, e):
        if dtype == "bf16":
            return bf16_decode(np.asarray(w[e]))
        if dtype == "mxfp4":
            return mx_dequantize(fp4_unpack(np.asarray(w[e])), np.asarray(scale[e]))
        return e4m3_decode(np.asarray(w[e])) * np.asarray(scale[e], dtype=np.float32)[:, None].astype(np.float64)

    flat = ids.reshape(-1)
    slot_tok = np.repeat(np.arange(T), k)
    computed = tok_mask[slot_tok]
    I = None
    out = np.full((T, D), np.nan)
    out[tok_mask] = 0.0
    contrib = np.full((T * k, D), np.nan)
    a_bits_all = None
    a_codes_all = None
    a_scale_all = None
    experts = np.unique(flat[computed])
    for e in experts:
        slots = np.nonzero((flat == e) & computed)[0]
        toks = slot_tok[slots]
        xh = dec_x(toks)                      # [n, D]
        W1 = dec_w(w1, w1_scale, e)           # [2I, D]
        if I is None:
            I = W1.shape[0] // 2
            a_bits_all = np.zeros((T * k, I), dtype=np.uint16)
            if dtype == "fp8":
                a_codes_all = np.zeros((T * k, I), dtype=np.uint8)
                a_scale_all = np.zeros(T * k, dtype=np.float32)
            elif dtype == "mxfp4":
                a_codes_all = np.zeros((T * k, I), dtype=np.uint8)
                a_scale_all = np.zeros((T * k, I // 32), dtype=np.uint8)
        gu = xh @ W1.T                        # [n, 2I]: gate then up
        g, u = gu[:, :I], gu[:, I:]
        a_bits = bf16_encode_rne(_silu(g) * u)
        a_bits_all[slots] = a_bits
        if dtype == "fp8":
            codes, sc, a_hat = requant_rows_fp8(a_bits)
            a_codes_all[slots] = codes
            a_scale_all[slots] = sc
        elif dtype == "mxfp4":
            codes, sc, a_hat = requant_rows_mx(a_bits)
            a_codes_all[slots] = codes
            a_scale_all[slots] = sc
        else:
            a_hat = bf16_decode(a_bits)
        W2 = dec_w(w2, w2_scale, e)           # [D, I]
        y = a_hat @ W2.T                      # [n, D]
        c = weights.reshape(-1)[slots].astype(np.float64)[:, None] * y
        contrib[slots] = c
        for r, t in enumerate(toks):
            out[t] += c[r]
    return LayerResult(out, contrib, a_bits_all, a_codes_all, a_scale_all, computed)
