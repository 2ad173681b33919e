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

from .codecs import (bf16_decode, bf16_encode_rne, e2m1_decode, e2m1_encode_rne_sat, e4m3_decode,
                     e4m3_encode_rne_sat, E4M3_MAX, fp4_unpack, MX_BLOCK, mx_dequantize, mx_quantize)


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


# Relative half-width of the fp32 evaluation of silu(g) * u around its exact value (an exp,
# a division and two products, each within a few fp32 units in the last place); 2^-20 is
# 16 such units.
SILU_REL = 2.0 ** -20


def _e4m3_spacing(m: np.ndarray) -> np.ndarray:
    """Spacing of e4m3 numbers at magnitude m (2^-9 in the subnormal range below 2^-6)."""
    _, e = np.frexp(np.maximum(np.abs(m), 2.0 ** -6))
    return np.ldexp(1.0, e - 4)


def _fp8_row_scale(amax: np.ndarray) -> np.ndarray:
    """Row scale of the fp8 requant: fp32(amax / 448), 1 for an all-zero row."""
    a32 = amax.astype(np.float32)
    return np.where(a32 > 0, a32 / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)


def _fp8_deq(v: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """e4m3 requant of bf16 values v with fp32 row scales, dequantised."""
    q = (v.astype(np.float32) / scale[:, None]).astype(np.float32)
    return e4m3_decode(e4m3_encode_rne_sat(q.astype(np.float64))) * scale[:, None].astype(np.float64)


def _mx_exp(amax: np.ndarray) -> np.ndarray:
    """MX block exponent (E8M0 code) of a block maximum: floor(log2 amax) - 2 + 127, 127 for 0."""
    _, ex = np.frexp(amax)
    return np.clip(np.where(amax > 0, ex - 1 - 2, 0) + 127, 0, 254)


def requant_spread(v: np.ndarray, a_bits: np.ndarray, band: np.ndarray, dtype: str):
    """Every intermediate a conforming implementation may produce, as a spread around the
    oracle's.

    v is the exact silu(g) * u (float64 [n, I]), a_bits its bf16 rounding (the oracle's a) and
    band the half-width of the interval around v that holds an implementation's value before
    its bf16 rounding (its GEMM accumulation and fp32 evaluation of silu).  Rounding is
    monotone, so that implementation's bf16 a lies in [lo, hi] = [bf16(v - band),
    bf16(v + band)].  Its requant follows the same rule as requant_rows_fp8 or
    requant_rows_mx on its own row:
    * fp8: the row scale lies in [scale(min amax), scale(max amax)]; with one scale possible,
      code = e4m3(a / scale) is monotone in a, so the dequantised value lies between those of
      lo and hi; otherwise it lies within half an e4m3 step (at its value) of its bf16 value;
    * mxfp4: likewise per block of 32 with the block exponent (E2M1 rounding error at most
      half a grid step, or 2 * scale for a value saturated at 6).
    Returns (lo, hi, spread, q_lo, q_hi): spread[n, i] bounds |a_hat_impl - a_hat_oracle|;
    q_lo/q_hi are the possible fp8 row scales (float32 [n]) or MX block exponents (uint8
    [n, I/32]); None for bf16."""
    a_ref = bf16_decode(a_bits)
    lo = bf16_decode(bf16_encode_rne(v - band))
    hi = bf16_decode(bf16_encode_rne(v + band))
    dev = np.maximum(np.abs(lo - a_ref), np.abs(hi - a_ref))
    if dtype == "bf16":
        return lo, hi, dev, None, None
    amin = np.where((lo <= 0) & (hi >= 0), 0.0, np.minimum(np.abs(lo), np.abs(hi)))
    amx = np.maximum(np.abs(lo), np.abs(hi))
    if dtype == "fp8":
        _, s_ref, ah_ref = requant_rows_fp8(a_bits)
        s_a, s_b = _fp8_row_scale(amin.max(axis=1)), _fp8_row_scale(amx.max(axis=1))
        q_lo, q_hi = np.minimum(s_a, s_b), np.maximum(s_a, s_b)
        fixed = (q_lo == q_hi)[:, None]
        sp_fixed = np.maximum(np.abs(_fp8_deq(lo, s_ref) - ah_ref), np.abs(_fp8_deq(hi, s_ref) - ah_ref))
        s_min, s_max = q_lo.astype(np.float64)[:, None], q_hi.astype(np.float64)[:, None]
        sp_var = dev + np.abs(a_ref - ah_ref) + 0.5 * _e4m3_spacing(amx / s_min) * s_max
        return lo, hi, np.where(fixed, sp_fixed, sp_var), q_lo, q_hi
    n, I = v.shape
    blk = lambda x: x.reshape(n, I // MX_BLOCK, MX_BLOCK)  # noqa: E731
    _, e_ref, ah_ref = requant_rows_mx(a_bits)
    e_a, e_b = _mx_exp(blk(amin).max(axis=2)), _mx_exp(blk(amx).max(axis=2))
    q_lo, q_hi = np.minimum(e_a, e_b).astype(np.uint8), np.maximum(e_a, e_b).astype(np.uint8)
    fixed = np.repeat(q_lo == q_hi, MX_BLOCK, axis=1)
    scale = np.repeat(np.ldexp(1.0, e_ref.astype(np.int64) - 127), MX_BLOCK, axis=1)
    deq = lambda x: e2m1_decode(e2m1_encode_rne_sat(x / scale)) * scale  # noqa: E731
    sp_fixed = np.maximum(np.abs(deq(lo) - ah_ref), np.abs(deq(hi) - ah_ref))
    s_max = np.repeat(np.ldexp(1.0, q_hi.astype(np.int64) - 127), MX_BLOCK, axis=1)
    sp_var = dev + np.abs(a_ref - ah_ref) + 2.0 * s_max
    return lo, hi, np.where(fixed, sp_fixed, sp_var), q_lo, q_hi


def _dsilu(z: np.ndarray) -> np.ndarray:
    """Derivative of silu: sigma(z) * (1 + z * (1 - sigma(z)))."""
    sg = 1.0 / (1.0 + np.exp(-z))
    return sg * (1.0 + z * (1.0 - sg))


@dataclass
class LayerResult:
    out: np.ndarray       # float64 [T, D]; rows not requested are NaN
    contrib: np.ndarray   # float64 [T*k, D]: routed-weighted down output of each slot
    a_bits: np.ndarray    # uint16 [T*k, I]: bf16 intermediate silu(g)*u (pre-requant)
    a_codes: np.ndarray | None   # uint8 [T*k, I]: fp8 codes, or mxfp4 codes (one per byte)
    a_scale: np.ndarray | None   # float32 [T*k] (fp8), or uint8 E8M0 [T*k, I/32] (mxfp4)
    computed: np.ndarray  # bool [T*k]: slots that were evaluated
    # float32 [T*k, I] (only with cond=True): first-order change of silu(g)*u when every
    # product x[d]*W1[e,n,d] of the gate and up sums is perturbed by its own magnitude,
    # |silu'(g) u| sum_d |W1[e,n,d] x[d]| + |silu(g)| sum_d |W1[e,I+n,d] x[d]|; times a
    # relative accumulation error it bounds how far the GEMM's rounding can move a.
    a_cond: np.ndarray | None = None
    # Only with band_rel (see moe_layer): the bf16 interval [a_lo, a_hi] holding an
    # implementation's intermediate, the spread of its requantised value around the oracle's
    # (requant_spread), the possible fp8 row scales or MX block exponents, and what those
    # alternatives can do to each slot row and token row after the down projection.
    a_lo: np.ndarray | None = None        # float32 [T*k, I]
    a_hi: np.ndarray | None = None        # float32 [T*k, I]
    a_spread: np.ndarray | None = None    # float32 [T*k, I]
    q_lo: np.ndarray | None = None        # fp8: float32 [T*k]; mxfp4: uint8 [T*k, I/32]
    q_hi: np.ndarray | None = None
    contrib_allow: np.ndarray | None = None  # float64 [T*k, D]: w_s * |W2| @ a_spread[s]
    out_allow: np.ndarray | None = None      # float64 [T, D]: sum of a token's contrib_allow


def moe_layer(x, w1, w2, ids, weights, dtype: str = "bf16", x_scale=None,
              w1_scale=None, w2_scale=None, tokens=None, slots=None, cond=False,
              band_rel=None) -> LayerResult:
    """Reference forward of one MoE layer.

    x: bf16 bits uint16 [T, D] (fp8: e4m3 codes uint8 [T, D] with x_scale fp32 [T];
       mxfp4: packed uint8 [T, D/2] with x_scale uint8 E8M0 [T, D/32]).
    w1: per-expert indexable, w1[e] is [2I, D] (bf16 bits or e4m3 codes with
        w1_scale[e] fp32 [2I]; mxfp4: packed [2I, D/2] with scales [2I, D/32]);
        w2[e] is [D, I] (with w2_scale[e] fp32 [D]; mxfp4: [D, I/2], [D, I/32]).
    ids int32 [T, k], weights fp32 [T, k] from routing.
    tokens: optional iterable of token indices to evaluate (others are NaN);
        only the experts those tokens use are read.
    slots: optional iterable of slot indices s = t*k + j evaluated as well (their
        contrib and intermediate rows; out only covers the tokens in `tokens`).
        With tokens=None and slots given, only those slots are evaluated.
    cond: also return a_cond (see LayerResult).
    band_rel: also return the alternatives of the intermediate (a_lo, a_hi, a_spread, q_lo,
        q_hi) and their effect on the outputs (contrib_allow, out_allow), for an
        implementation whose gate-up sums have relative error band_rel with respect to their
        sums of |products| (band = band_rel * a_cond + SILU_REL * |silu(g) u|).
    """
    if band_rel is not None:
        cond = True
    if dtype not in ("bf16", "fp8", "mxfp4"):
        raise ValueError("dtype must be 'bf16', 'fp8' or 'mxfp4'")
    ids = np.asarray(ids, dtype=np.int64)
    weights = np.asarray(weights, dtype=np.float32)
    T, k = ids.shape
    D = np.asarray(x).shape[1] * (2 if dtype == "mxfp4" else 1)
    tok_mask = np.zeros(T, dtype=bool)
    if tokens is None and slots is None:
        tok_mask[:] = True
    elif tokens is not None:
        tok_mask[np.asarray(list(tokens), dtype=np.int64)] = True
    slot_mask = np.zeros(T * k, dtype=bool)
    if slots is not None:
        slot_mask[np.asarray(list(slots), dtype=np.int64)] = True

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
    computed = tok_mask[slot_tok] | slot_mask
    I = None
    a_cond_all = None
    a_lo_all = a_hi_all = a_spread_all = q_lo_all = q_hi_all = contrib_allow = out_allow = None
    out = np.full((T, D), np.nan)
    out[tok_mask] = 0.0
    contrib = np.full((T * k, D), np.nan)
    a_bits_all = None
    a_codes_all = None
    a_scale_all = None
    experts = np.unique(flat[computed])
    for e in experts:
        sl = np.nonzero((flat == e) & computed)[0]
        toks = slot_tok[sl]
        xh = dec_x(toks)                      # [n, D]
        W1 = dec_w(w1, w1_scale, e)           # [2I, D]
        if I is None:
            I = W1.shape[0] // 2
            a_bits_all = np.zeros((T * k, I), dtype=np.uint16)
            if cond:
                a_cond_all = np.zeros((T * k, I), dtype=np.float32)
            if band_rel is not None:
                a_lo_all = np.zeros((T * k, I), dtype=np.float32)
                a_hi_all = np.zeros((T * k, I), dtype=np.float32)
                a_spread_all = np.zeros((T * k, I), dtype=np.float32)
                contrib_allow = np.zeros((T * k, D))
                out_allow = np.zeros((T, D))
                if dtype == "fp8":
                    q_lo_all = np.zeros(T * k, dtype=np.float32)
                    q_hi_all = np.zeros(T * k, dtype=np.float32)
                elif dtype == "mxfp4":
                    q_lo_all = np.zeros((T * k, I // MX_BLOCK), dtype=np.uint8)
                    q_hi_all = np.zeros((T * k, I // MX_BLOCK), dtype=np.uint8)
            if dtype == "fp8":
                a_codes_all = np.zeros((T * k, I), dtype=np.uint8)
                a_scale_all = np.zeros(T * k, dtype=np.float32)
            elif dtype == "mxfp4":
                a_codes_all = np.zeros((T * k, I), dtype=np.uint8)
                a_scale_all = np.zeros((T * k, I // 32), dtype=np.uint8)
        gu = xh @ W1.T                        # [n, 2I]: gate then up
        g, u = gu[:, :I], gu[:, I:]
        v = _silu(g) * u
        a_bits = bf16_encode_rne(v)
        a_bits_all[sl] = a_bits
        if cond:
            gu_abs = np.abs(xh) @ np.abs(W1).T  # [n, 2I]: sum of |products| of each sum
            a_cond = np.abs(_dsilu(g) * u) * gu_abs[:, :I] + np.abs(_silu(g)) * gu_abs[:, I:]
            a_cond_all[sl] = a_cond
        if band_rel is not None:
            band = band_rel * a_cond + SILU_REL * np.abs(v)
            lo, hi, spread, qlo, qhi = requant_spread(v, a_bits, band, dtype)
            a_lo_all[sl], a_hi_all[sl], a_spread_all[sl] = lo, hi, spread
            if qlo is not None:
                q_lo_all[sl], q_hi_all[sl] = qlo, qhi
        if dtype == "fp8":
            codes, sc, a_hat = requant_rows_fp8(a_bits)
            a_codes_all[sl] = codes
            a_scale_all[sl] = sc
        elif dtype == "mxfp4":
            codes, sc, a_hat = requant_rows_mx(a_bits)
            a_codes_all[sl] = codes
            a_scale_all[sl] = sc
        else:
            a_hat = bf16_decode(a_bits)
        W2 = dec_w(w2, w2_scale, e)           # [D, I]
        y = a_hat @ W2.T                      # [n, D]
        w_sl = weights.reshape(-1)[sl].astype(np.float64)[:, None]
        c = w_sl * y
        contrib[sl] = c
        if band_rel is not None:
            ca = np.abs(w_sl) * (a_spread_all[sl].astype(np.float64) @ np.abs(W2).T)
            contrib_allow[sl] = ca
        for r, t in enumerate(toks):
            if tok_mask[t]:
                out[t] += c[r]
                if band_rel is not None:
                    out_allow[t] += ca[r]
    return LayerResult(out, contrib, a_bits_all, a_codes_all, a_scale_all, computed, a_cond_all,
                       a_lo_all, a_hi_all, a_spread_all, q_lo_all, q_hi_all, contrib_allow, out_allow)
