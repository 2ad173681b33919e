"""Pins of the layer oracle: pure-Python brute force, dense SwiGLU special case, invariances."""

import math

import numpy as np
import pytest
import torch

import synth
from oracle import bf16_decode, bf16_encode_rne, e4m3_decode, moe_layer, route
from oracle.layer import requant_rows_fp8


def np_inputs(inp):
    out = {}
    for key, v in inp.items():
        if v.dtype == torch.bfloat16:
            out[key] = v.view(torch.int16).numpy().view(np.uint16)
        else:
            out[key] = v.numpy()
    return out


def bf16_round_torch(v: float) -> float:
    return float(torch.tensor(v, dtype=torch.float32).to(torch.bfloat16).float())


FP4_VALUES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]  # E2M1 magnitudes (MX format)


def fp4_value(byte_row, i):
    """Element i of a packed row (element 2j in the low nibble)."""
    code = (byte_row[i // 2] >> (4 * (i % 2))) & 0xF
    return -FP4_VALUES[code & 7] if code & 8 else FP4_VALUES[code & 7]


def mx_round_block(vals):
    """One MX block of 32 values: scale 2**(floor(log2 amax) - 2), elements to the nearest
    E2M1 magnitude (ties to the even code), clamped at 6; returns the dequantised values."""
    amax = max(abs(v) for v in vals)
    if amax == 0:
        return [0.0] * len(vals)
    scale = 2.0 ** (math.frexp(amax)[1] - 1 - 2)
    out = []
    for v in vals:
        y = min(abs(v) / scale, 6.0)
        best = min(range(8), key=lambda c: (abs(y - FP4_VALUES[c]), c % 2))
        out.append(math.copysign(FP4_VALUES[best], v) * scale)
    return out


def brute_layer(x, w1, w2, ids, wts, dtype="bf16", xs=None, w1s=None, w2s=None):
    """Pure-Python loops over tokens, slots, channels; rounding by torch's casts."""
    T, k = ids.shape
    D = len(x[0]) * (2 if dtype == "mxfp4" else 1)
    I = len(w1[0]) // 2

    def xv(t, d):
        if dtype == "mxfp4":
            return fp4_value(x[t], d) * 2.0 ** (int(xs[t][d // 32]) - 127)
        if dtype == "bf16":
            return float(torch.tensor(int(x[t][d]), dtype=torch.int32).to(torch.int16).view(torch.bfloat16))
        return float(torch.tensor(int(x[t][d]), dtype=torch.uint8).view(torch.float8_e4m3fn)) * float(xs[t])

    def wv(w, s, e, r, c):
        if dtype == "mxfp4":
            return fp4_value(w[e][r], c) * 2.0 ** (int(s[e][r][c // 32]) - 127)
        if dtype == "bf16":
            return float(torch.tensor(int(w[e][r][c]), dtype=torch.int32).to(torch.int16).view(torch.bfloat16))
        return float(torch.tensor(int(w[e][r][c]), dtype=torch.uint8).view(torch.float8_e4m3fn)) * float(s[e][r])

    out = [[0.0] * D for _ in range(T)]
    for t in range(T):
        for j in range(k):
            e = int(ids[t][j])
            a = []
            for n in range(I):
                g = sum(wv(w1, w1s, e, n, d) * xv(t, d) for d in range(D))
                u = sum(wv(w1, w1s, e, I + n, d) * xv(t, d) for d in range(D))
                a.append(bf16_round_torch(g / (1.0 + math.exp(-g)) * u))
            if dtype == "fp8":
                amax = max(abs(v) for v in a)
                sc = float(np.float32(amax) / np.float32(448.0)) if amax > 0 else 1.0
                q = torch.tensor([v / sc for v in a], dtype=torch.float32)
                q = (q.float() / 1.0).to(torch.float8_e4m3fn).float().tolist()
                a = [v * sc for v in q]
            if dtype == "mxfp4":
                a = [v for b in range(0, I, 32) for v in mx_round_block(a[b:b + 32])]
            for d in range(D):
                y = sum(wv(w2, w2s, e, d, n) * a[n] for n in range(I))
                out[t][d] += float(wts[t][j]) * y
    return np.array(out)


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "mxfp4"])
@pytest.mark.parametrize("seed", [0, 1])
def test_brute_force_tiny(dtype, seed):
    # MX blocks need multiples of 32 along K
    T, E, k, D, I = (3, 4, 2, 8, 4) if dtype != "mxfp4" else (3, 4, 2, 64, 32)
    inp = np_inputs(synth.small_layer_inputs(T, E, k, D, I, dtype, seed=seed, w_std=0.3))
    r = route(inp["logits"], k, 16)
    ref = moe_layer(inp["x"], inp["w1"], inp["w2"], r.ids, r.weights, dtype,
                    inp.get("x_scale"), inp.get("w1_scale"), inp.get("w2_scale"))
    bf = brute_layer(inp["x"].tolist(), inp["w1"].tolist(), inp["w2"].tolist(), r.ids, r.weights,
                     dtype, inp.get("x_scale"), inp.get("w1_scale"), inp.get("w2_scale"))
    assert np.allclose(ref.out, bf, rtol=1e-12, atol=1e-12 * np.abs(bf).max())


def test_dense_swiglu_special_case():
    # E = 1, k = 1: every token goes to the one expert with weight 1.0 -> a dense SwiGLU FFN.
    T, D, I = 5, 64, 32
    inp = synth.small_layer_inputs(T, 1, 1, D, I, "bf16", seed=3, w_std=0.1)
    npi = np_inputs(inp)
    r = route(npi["logits"], 1, 16)
    assert np.all(r.weights == 1.0)
    res = moe_layer(npi["x"], npi["w1"], npi["w2"], r.ids, r.weights)
    x = inp["x"].double()
    w1 = inp["w1"][0].double()
    w2 = inp["w2"][0].double()
    gu = x @ w1.T
    act = torch.nn.functional.silu(gu[:, :I]) * gu[:, I:]
    a_ref = act.to(torch.bfloat16)
    a_ours = torch.from_numpy(bf16_decode(res.a_bits)).to(torch.bfloat16)
    # the bf16 intermediate: identical up to rare 1-ulp double-rounding cases of torch's cast
    mism = (a_ref != a_ours).sum().item()
    assert mism <= max(1, a_ref.numel() // 1000)
    # second GEMM + combine: exact in fp64 given the oracle's intermediate
    out_ref = torch.from_numpy(bf16_decode(res.a_bits)) @ w2.T
    assert torch.allclose(torch.from_numpy(res.out), out_ref, rtol=1e-12, atol=1e-14)
    # and against the fully independent dense chain
    out_dense = a_ref.double() @ w2.T
    rms = out_dense.pow(2).mean().sqrt()
    assert (torch.from_numpy(res.out) - out_dense).abs().max() <= 1e-2 * rms


def test_expert_relabel_invariance():
    T, E, k, D, I = 6, 8, 3, 32, 16
    npi = np_inputs(synth.small_layer_inputs(T, E, k, D, I, "bf16", seed=5))
    r = route(npi["logits"], k, 16)
    base = moe_layer(npi["x"], npi["w1"], npi["w2"], r.ids, r.weights).out
    perm = np.random.default_rng(0).permutation(E)
    inv = np.argsort(perm)
    # expert e in the new labelling is old expert perm[e]
    l2 = npi["logits"][:, perm]
    r2 = route(l2, k, 16)
    assert np.array_equal(perm[r2.ids], r.ids)  # no ties -> same picks
    out2 = moe_layer(npi["x"], npi["w1"][perm], npi["w2"][perm], r2.ids, r2.weights).out
    assert np.allclose(out2, base, rtol=1e-12, atol=1e-14)
    del inv


def test_zeroing_one_expert_removes_exactly_its_slots():
    T, E, k, D, I = 8, 6, 2, 32, 16
    npi = np_inputs(synth.small_layer_inputs(T, E, k, D, I, "bf16", seed=7))
    r = route(npi["logits"], k, 16)
    full = moe_layer(npi["x"], npi["w1"], npi["w2"], r.ids, r.weights)
    e0 = int(r.ids[0, 0])
    w2 = npi["w2"].copy()
    w2[e0] = 0
    cut = moe_layer(npi["x"], npi["w1"], w2, r.ids, r.weights)
    expect = full.out.copy()
    flat = r.ids.reshape(-1)
    for s in np.nonzero(flat == e0)[0]:
        expect[s // k] -= full.contrib[s]
    assert np.allclose(cut.out, expect, rtol=1e-12, atol=1e-13)


def test_one_hot_weights_recover_slot_outputs():
    T, E, k, D, I = 4, 5, 2, 16, 8
    npi = np_inputs(synth.small_layer_inputs(T, E, k, D, I, "bf16", seed=9))
    r = route(npi["logits"], k, 16)
    ones = np.zeros_like(r.weights)
    ones[:, 1] = 1.0  # only the second pick counts: catches a gather that reads slot 0
    res = moe_layer(npi["x"], npi["w1"], npi["w2"], r.ids, ones)
    for t in range(T):
        e = r.ids[t, 1]
        a = bf16_decode(res.a_bits[t * k + 1])
        y = bf16_decode(npi["w2"][e]) @ a
        assert np.allclose(res.out[t], y, rtol=1e-12, atol=1e-14)
    assert not np.allclose(res.out, moe_layer(npi["x"], npi["w1"], npi["w2"], r.ids,
                                               ones[:, ::-1].copy()).out)


def test_fp8_requant_rule():
    rng = np.random.default_rng(11)
    a = rng.standard_normal((40, 64)).astype(np.float32)
    a[3] = 0.0
    bits = a.astype(np.float32).view(np.uint32)
    a_bits = ((bits + np.uint32(0x8000)) >> np.uint32(16)).astype(np.uint16)  # any bf16 values
    codes, scale, deq = requant_rows_fp8(a_bits)
    a32 = torch.from_numpy((a_bits.astype(np.uint32) << 16).view(np.float32))
    amax = a32.abs().amax(1)
    ref_scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    assert np.array_equal(scale, ref_scale.numpy())
    ref_codes = (a32 / ref_scale[:, None]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref_codes)
    assert np.all(np.abs(e4m3_decode(codes)).max(1)[np.arange(40) != 3] == 448.0)  # row max maps to 448
    assert np.all(deq[3] == 0) and scale[3] == 1.0
    # dequantised values within half an e4m3 step (relative 2**-4) of the bf16 input
    rel = np.abs(deq - a32.double().numpy()) / np.maximum(np.abs(a32.double().numpy()), 2.0**-6 * scale[:, None])
    assert rel.max() <= 2.0**-4 + 1e-12


def test_token_subset_reads_only_needed_experts():
    T, E, k, D, I = 10, 12, 2, 16, 8
    npi = np_inputs(synth.small_layer_inputs(T, E, k, D, I, "bf16", seed=13))
    r = route(npi["logits"], k, 16)
    full = moe_layer(npi["x"], npi["w1"], npi["w2"], r.ids, r.weights)
    used = set(r.ids[[2, 7]].reshape(-1).tolist())
    w1 = {e: npi["w1"][e] for e in used}
    w2 = {e: npi["w2"][e] for e in used}
    part = moe_layer(npi["x"], w1, w2, r.ids, r.weights, tokens=[2, 7])
    assert np.array_equal(part.out[[2, 7]], full.out[[2, 7]])
    assert np.isnan(part.out[0]).all()


def test_slot_subset_matches_full():
    """slots= evaluates exactly the listed slots: their contrib and intermediate rows equal the
    full evaluation's, and no token output is formed."""
    T, E, k, D, I = 10, 12, 3, 16, 8
    npi = np_inputs(synth.small_layer_inputs(T, E, k, D, I, "fp8", seed=5))
    r = route(npi["logits"], k, 16)
    kw = dict(x_scale=npi["x_scale"], w1_scale=npi["w1_scale"], w2_scale=npi["w2_scale"])
    full = moe_layer(npi["x"], npi["w1"], npi["w2"], r.ids, r.weights, "fp8", **kw)
    sl = [1, 4, 17, 29]
    part = moe_layer(npi["x"], npi["w1"], npi["w2"], r.ids, r.weights, "fp8", slots=sl, **kw)
    # fp64 BLAS may block a product of fewer rows differently: equal to rounding
    assert np.allclose(part.contrib[sl], full.contrib[sl], rtol=1e-12, atol=0)
    assert np.array_equal(part.a_codes[sl], full.a_codes[sl])
    assert np.array_equal(part.computed, np.isin(np.arange(T * k), sl))
    assert np.isnan(part.out).all()
    both = moe_layer(npi["x"], npi["w1"], npi["w2"], r.ids, r.weights, "fp8", tokens=[2], slots=[0], **kw)
    assert np.allclose(both.out[2], full.out[2], rtol=1e-12, atol=0) and np.isnan(both.out[0]).all()
    assert np.allclose(both.contrib[0], full.contrib[0], rtol=1e-12, atol=0)


def test_a_cond_brute_force():
    """a_cond against a pure-Python loop: the sums of |products| of the gate and up rows, with
    silu's derivative taken by a central difference."""
    T, E, k, D, I = 3, 4, 2, 8, 4
    npi = np_inputs(synth.small_layer_inputs(T, E, k, D, I, "bf16", seed=9, w_std=0.3))
    r = route(npi["logits"], k, 16)
    res = moe_layer(npi["x"], npi["w1"], npi["w2"], r.ids, r.weights, cond=True)
    x = bf16_decode(npi["x"])
    silu = lambda z: z / (1.0 + math.exp(-z))  # noqa: E731
    for t in range(T):
        for j in range(k):
            e = int(r.ids[t, j])
            W = bf16_decode(npi["w1"][e])
            for n in range(I):
                g = sum(float(W[n, d]) * float(x[t, d]) for d in range(D))
                u = sum(float(W[I + n, d]) * float(x[t, d]) for d in range(D))
                ag = sum(abs(float(W[n, d]) * float(x[t, d])) for d in range(D))
                au = sum(abs(float(W[I + n, d]) * float(x[t, d])) for d in range(D))
                h = 1e-5
                ds = (silu(g + h) - silu(g - h)) / (2 * h)
                want = abs(ds * u) * ag + abs(silu(g)) * au
                got = float(res.a_cond[t * k + j, n])
                assert abs(got - want) <= 1e-5 * want + 1e-30, (t, j, n, got, want)


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "mxfp4"])
def test_requant_spread_covers_every_alternative(dtype):
    """Alternative implementations: each slot's silu(g)*u moved anywhere inside the band
    (random points and both ends), rounded to bf16 and requantised by the same rule.  Their
    bf16 rows lie in [a_lo, a_hi], their scales in [q_lo, q_hi], their dequantised rows within
    a_spread of the oracle's, and their slot and token outputs within contrib_allow and
    out_allow.  A wide band (2^-9, 2^-7) makes scale and exponent changes happen too."""
    from oracle.layer import SILU_REL, requant_rows_fp8, requant_rows_mx
    from oracle import mx_dequantize
    T, E, k, D, I = 24, 3, 2, 64, 128
    band_rel = {"bf16": 2.0 ** -9, "fp8": 2.0 ** -9, "mxfp4": 2.0 ** -7}[dtype]
    npi = np_inputs(synth.small_layer_inputs(T, E, k, D, I, dtype, seed=17, w_std=0.3))
    r = route(npi["logits"], k, 16)
    kw = {} if dtype == "bf16" else dict(x_scale=npi["x_scale"], w1_scale=npi["w1_scale"],
                                         w2_scale=npi["w2_scale"])
    res = moe_layer(npi["x"], npi["w1"], npi["w2"], r.ids, r.weights, dtype, band_rel=band_rel, **kw)

    def dec(w, sc, e):
        if dtype == "bf16":
            return bf16_decode(w[e])
        if dtype == "fp8":
            return e4m3_decode(w[e]) * sc[e][:, None].astype(np.float64)
        from oracle import fp4_unpack
        return mx_dequantize(fp4_unpack(w[e]), sc[e])

    if dtype == "bf16":
        xh = bf16_decode(npi["x"])
    elif dtype == "fp8":
        xh = e4m3_decode(npi["x"]) * npi["x_scale"][:, None].astype(np.float64)
    else:
        from oracle import fp4_unpack
        xh = mx_dequantize(fp4_unpack(npi["x"]), npi["x_scale"])
    flat = r.ids.reshape(-1)
    v = np.zeros((T * k, I))
    for s_ in range(T * k):
        W1 = dec(npi["w1"], npi.get("w1_scale"), flat[s_])
        gu = W1 @ xh[s_ // k]
        g, u = gu[:I], gu[I:]
        v[s_] = g / (1 + np.exp(-g)) * u
    band = band_rel * res.a_cond.astype(np.float64) + SILU_REL * np.abs(v)
    if dtype == "fp8":
        ah_ref = requant_rows_fp8(res.a_bits)[2]
    elif dtype == "mxfp4":
        ah_ref = requant_rows_mx(res.a_bits)[2]
    else:
        ah_ref = bf16_decode(res.a_bits)
    rng = np.random.default_rng(0)
    var_seen = False
    for trial in range(40):
        f = {0: -1.0, 1: 1.0}.get(trial, None)
        shift = f * band if f is not None else rng.uniform(-1, 1, band.shape) * band
        alt_bits = bf16_encode_rne(v + shift)
        alt = bf16_decode(alt_bits)
        assert np.all(alt >= res.a_lo) and np.all(alt <= res.a_hi)
        if dtype == "fp8":
            _, sc, ah = requant_rows_fp8(alt_bits)
            assert np.all(sc >= res.q_lo) and np.all(sc <= res.q_hi)
        elif dtype == "mxfp4":
            _, sc, ah = requant_rows_mx(alt_bits)
            assert np.all(sc >= res.q_lo) and np.all(sc <= res.q_hi)
        else:
            ah = alt
        assert np.all(np.abs(ah - ah_ref) <= res.a_spread.astype(np.float64) * (1 + 1e-6) + 1e-30)
        out = np.zeros((T, D))
        for s_ in range(T * k):
            W2 = dec(npi["w2"], npi.get("w2_scale"), flat[s_])
            c = float(r.weights.reshape(-1)[s_]) * (W2 @ ah[s_])
            assert np.all(np.abs(c - res.contrib[s_]) <= res.contrib_allow[s_] * (1 + 1e-9) + 1e-12)
            out[s_ // k] += c
        assert np.all(np.abs(out - res.out) <= res.out_allow * (1 + 1e-9) + 1e-12)
    if dtype != "bf16":
        var_seen = bool(np.any(res.q_lo != res.q_hi))
        assert var_seen, "the band never moved a scale: the wide-band branch went untested"
    assert (res.a_spread > 0).any()
