"""Helpers for the GPU parity tests: host copies for the oracle and the comparison rules."""

from __future__ import annotations

import numpy as np
import torch

import oracle

BF16_TOL = 2e-2     # max|err| <= 2e-2 * rms(out), and cosine >= 0.9999
BF16_COS = 0.9999
FP8_TOL = 5e-2      # max|err| <= 5e-2 * rms(out)
W_REL = 1e-6        # routing weights: fp32 relative error


def host_bits(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy array of its stored bits (bf16 -> uint16, uint8 stays uint8)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class PerExpert:
    """Indexable per expert; copies one expert's slab to the host on demand."""

    def __init__(self, t: torch.Tensor):
        self.t = t

    def __getitem__(self, e):
        return host_bits(self.t[int(e)])


def oracle_route(logits: torch.Tensor, k: int, B: int, score="softmax", renorm=True):
    return oracle.route(logits.detach().cpu().numpy(), k, B, score, renorm)


def check_route(got: dict, ref, T: int, k: int):
    """Bit-exact ids, sort, expert ids and num_valid; weights within fp32 rel 1e-6."""
    nv = int(got["num_valid"].item())
    assert nv == ref.num_valid, f"num_valid {nv} != {ref.num_valid}"
    if T == 0:
        return
    ids = got["topk_ids"].cpu().numpy()
    bad = np.argwhere(ids != ref.ids)
    assert bad.size == 0, f"topk_ids differ at {bad[:5].tolist()}: got {ids[tuple(bad[0])]} want {ref.ids[tuple(bad[0])]}"
    sid = got["sorted_token_ids"].cpu().numpy()
    assert np.array_equal(sid[: ref.cap], ref.sorted_token_ids), \
        f"sorted ids differ at {np.nonzero(sid[:ref.cap] != ref.sorted_token_ids)[0][:8].tolist()}"
    eid = got["expert_ids"].cpu().numpy()
    assert np.array_equal(eid[: len(ref.expert_ids)], ref.expert_ids), \
        f"expert ids differ at {np.nonzero(eid[:len(ref.expert_ids)] != ref.expert_ids)[0][:8].tolist()}"
    w = got["topk_weights"].cpu().numpy().astype(np.float64)
    wr = ref.weights.astype(np.float64)
    # relative 1e-6; an fp32 subnormal weight may sit one subnormal step (2^-149) away
    excess = np.abs(w - wr) - (W_REL * np.abs(wr) + 2.0 ** -149)
    rel = np.abs(w - wr) / np.maximum(np.abs(wr), 1e-45)
    assert excess.max() <= 0, f"weights rel err {rel.max():.3g} at {np.unravel_index(rel.argmax(), rel.shape)}"


def take_rows(t: torch.Tensor, rows) -> np.ndarray:
    """Rows of a device tensor as float64 on the host (gathered on the device first)."""
    idx = torch.as_tensor(np.asarray(rows, dtype=np.int64), device=t.device)
    return t.detach().index_select(0, idx).float().cpu().double().numpy()


def _within(got: np.ndarray, ref: np.ndarray, tol: float, cos_min, allow):
    """|got - ref| <= tol * rms(ref) + allow element by element (allow: the oracle's room for
    the intermediate's rounding decisions, or None); cosine >= cos_min.  Returns max|err|/rms,
    the cosine and max(allow)/rms."""
    assert np.isfinite(got).all()
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = np.abs(got - ref)
    room = tol * rms + (0.0 if allow is None else allow)
    cos = float((got * ref).sum() / (np.linalg.norm(got) * np.linalg.norm(ref) + 1e-300))
    i = np.unravel_index(np.argmax(err - room), err.shape)
    extra = "" if allow is None else f" + allowance {allow[i]:.4g}"
    assert np.all(err <= room), (f"|err| {err[i]:.4g} at {i} > {tol} * rms {rms:.4g}{extra} "
                                 f"(max|err|/rms {err.max() / rms:.4g}); cos {cos:.6f}")
    if cos_min is not None:
        assert cos >= cos_min, f"cosine {cos:.7f} < {cos_min}"
    return float(err.max()) / rms, cos, (0.0 if allow is None else float(np.max(allow)) / rms)


def compare_out(out_gpu: torch.Tensor, ref_out: np.ndarray, rows, tol: float, cos_min: float | None,
                allow: np.ndarray | None = None):
    """max|err| <= tol * rms(ref) (+ allow[rows]) over the given rows, cosine >= cos_min."""
    return _within(take_rows(out_gpu, rows), ref_out[rows], tol, cos_min,
                   None if allow is None else allow[rows])


def combined_fp32(y: torch.Tensor, mode: str, k: int, rows) -> np.ndarray:
    """The fp32 value the combine rounds to bf16, for the given token rows: ATOMIC, the fp32
    accumulator row; REDUCE, the token's k slot rows added in fp32 from 0, slot 0 first (the
    order of the reduction kernel)."""
    rows = np.asarray(rows, dtype=np.int64)
    if mode == "atomic":
        return take_rows(y, rows).astype(np.float32)
    slots = (rows[:, None] * k + np.arange(k)[None, :]).reshape(-1)
    ys = take_rows(y, slots).astype(np.float32).reshape(len(rows), k, -1)
    acc = np.zeros(ys[:, 0].shape, dtype=np.float32)
    for j in range(k):
        acc = (acc + ys[:, j]).astype(np.float32)
    return acc


# Half a bf16 step relative to the value rounded: bf16 keeps 8 significant bits, so round to
# nearest even moves a value by at most 2^-8 of its magnitude.
BF16_HALF_STEP = 2.0 ** -8


def contrib_magnitude(ref, rows, k: int, tol: float) -> np.ndarray:
    """[len(rows), D]: sum over a token's k slots of |c_j| plus the room the slot-row checks
    give the kernel's fp32 contribution (tol * rms of those contributions + the oracle's
    contrib_allow): a bound on sum_j |c~_j| for the kernel's own contributions c~_j, the
    magnitude a bf16 rounding of each of them is measured against."""
    rows = np.asarray(rows, dtype=np.int64)
    D = ref.contrib.shape[1]
    c = ref.contrib.reshape(-1, k, D)[rows]
    rms_c = float(np.sqrt(np.mean(c * c)))
    room = tol * rms_c + (0.0 if ref.contrib_allow is None else ref.contrib_allow.reshape(-1, k, D)[rows])
    return (np.abs(c) + room).sum(axis=1)


def compare_layer(out: torch.Tensor, y: torch.Tensor, mode: str, k: int, ref, rows,
                  tol: float, cos_min: float | None):
    """Layer output of the modes with a separate combine, in two parts: the bf16 output is the
    fp32 combined value rounded to nearest even, bit for bit; the fp32 value is within
    tol * rms(out) of the oracle's exact sum (and cosine >= cos_min).  The bound applies before
    the output's own rounding, which alone moves an element by up to half a bf16 step (more
    than 2e-2 * rms for elements beyond 8 * rms).  ref is the oracle's LayerResult; its
    out_allow (room for the intermediate's rounding decisions) is added element by element.
    reduce_bf16: each slot row was rounded to bf16 once before the sum, which adds half a bf16
    step of each contribution, 2^-8 * contrib_magnitude."""
    pre = combined_fp32(y, mode, k, rows)
    got_bits = host_bits(out)[np.asarray(rows, dtype=np.int64)]
    want_bits = oracle.bf16_encode_rne(pre.astype(np.float64))
    bad = np.argwhere(got_bits != want_bits)
    assert bad.size == 0, (f"output is not the rounded fp32 combine at {bad[:4].tolist()}: "
                           f"{got_bits[tuple(bad[0])]:#06x} vs {want_bits[tuple(bad[0])]:#06x}")
    allow = None if ref.out_allow is None else ref.out_allow[rows]
    if mode == "reduce_bf16":
        extra = BF16_HALF_STEP * contrib_magnitude(ref, rows, k, tol)
        allow = extra if allow is None else allow + extra
    return _within(pre.astype(np.float64), ref.out[rows], tol, cos_min, allow)


def compare_slot_rows(y: torch.Tensor, mode: str, ref, slots, tol: float, cos_min: float | None):
    """Reduce-mode slot rows against the oracle's contributions, under the output's bounds
    plus the oracle's contrib_allow; bf16 slot rows also move by up to half a bf16 step of
    the kernel's fp32 contribution, at most 2^-8 * (|c| + the fp32 room)."""
    slots = np.asarray(slots, dtype=np.int64)
    want = ref.contrib[slots]
    allow = None if ref.contrib_allow is None else ref.contrib_allow[slots]
    if mode == "reduce_bf16":
        rms = float(np.sqrt(np.mean(want * want)))
        room = tol * rms + (0.0 if allow is None else allow)
        extra = BF16_HALF_STEP * (np.abs(want) + room)
        allow = extra if allow is None else allow + extra
    return _within(take_rows(y, slots), want, tol, cos_min, allow)


def compare_out_bf16_atomic(out_gpu: torch.Tensor, ref, rows, k: int, tol: float):
    """Packed bf16 atomic accumulation: each of a token's k contributions is rounded to bf16
    and each of the k atomic adds rounds the running sum to bf16, so on top of the fp32
    modes' bound tol * rms(ref) an element may move by (k + 1) half bf16 steps, each at most
    2^-8 of a value no larger than M = sum_j |c~_j| (1 + 2^-8)^k (the kernel's fp32
    contributions, bounded by contrib_magnitude; the factor covers the running sum's own
    roundings).  ref is the oracle's LayerResult.  Returns the largest fraction of that
    allowance used."""
    got = take_rows(out_gpu, rows)
    ref_o = ref.out[rows]
    assert np.isfinite(got).all()
    rms = float(np.sqrt(np.mean(ref_o * ref_o)))
    m_abs = contrib_magnitude(ref, rows, k, tol) * (1.0 + BF16_HALF_STEP) ** k
    allow = tol * rms + (k + 1) * BF16_HALF_STEP * m_abs
    if ref.out_allow is not None:
        allow = allow + ref.out_allow[rows]
    err = np.abs(got - ref_o)
    used = float((err / allow).max())
    i = np.unravel_index(np.argmax(err / allow), err.shape)
    assert used <= 1.0, (f"err {err[i]:.4g} > allowance {allow[i]:.4g} at {i} (ref {ref_o[i]:.5g}, "
                         f"sum|c| bound {m_abs[i]:.4g}, rms {rms:.4g})")
    return used


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |v| (normal range)."""
    _, e = np.frexp(np.maximum(np.abs(v), 2.0 ** -126))
    return np.ldexp(1.0, e - 8)


# Relative error of the gate-up GEMM's sums with respect to their sum of |products|: sixteen
# times the largest value tests/test_gpu_accumulation.py measured on gfx950 (sums of 7168
# products that cancel exactly but round differently, decode and prefill kernels: bf16
# 6.5e-8, fp8 1.1e-6, mxfp4 0, its block-scaled E2M1 sums being exact in fp32), rounded up to
# a power of two; mxfp4 (the same MFMA instruction family) takes fp8's.  The oracle turns it
# into the interval that holds the kernels' intermediate and into what the requant decisions
# inside that interval can do to the outputs (oracle.moe_layer(band_rel=...)).
ACC_REL = {"bf16": 2.0 ** -19, "fp8": 2.0 ** -15, "mxfp4": 2.0 ** -15}


def check_a_bf16(got: np.ndarray, ref, rows):
    """bf16 intermediate, element by element: inside the oracle's interval [a_lo, a_hi] (the
    bf16 roundings of every value the accumulation band allows).  Diagnostic as well: at most
    1% of the elements more than one bf16 step from the oracle's a."""
    lo, hi = ref.a_lo[rows].astype(np.float64), ref.a_hi[rows].astype(np.float64)
    out = (got < lo) | (got > hi)
    if out.any():
        i = tuple(np.argwhere(out)[0])
        raise AssertionError(f"intermediate {got[i]:.6g} at {i} outside [{lo[i]:.6g}, {hi[i]:.6g}]")
    want = oracle.bf16_decode(ref.a_bits[rows])
    frac = float(np.mean(np.abs(got - want) > bf16_ulp(want) * 1.0001))
    assert frac <= 0.01, f"{frac:.4f} of the bf16 intermediate is more than 1 ulp off"


def _spread_check(deq_got, deq_want, spread, what):
    d = np.abs(deq_got - deq_want)
    allow = spread.astype(np.float64) * (1 + 1e-6)
    bad = d > allow
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what} value {deq_got[i]:.6g} vs {deq_want[i]:.6g} at {i}: "
                             f"diff {d[i]:.4g} > spread {allow[i]:.4g}")


def check_a_fp8(codes_got, scale_got, ref, rows):
    """fp8 intermediate, element by element: the row scale inside the oracle's possible range
    and every dequantised value within the oracle's spread (requant decisions taken on any
    bf16 row the accumulation band allows).  Diagnostic as well: at most 2% of the codes
    differ."""
    assert np.all((scale_got >= ref.q_lo[rows]) & (scale_got <= ref.q_hi[rows])), "a_scale outside its range"
    from oracle import e4m3_decode
    got = e4m3_decode(codes_got) * scale_got.astype(np.float64)[:, None]
    want = e4m3_decode(ref.a_codes[rows]) * ref.a_scale[rows].astype(np.float64)[:, None]
    _spread_check(got, want, ref.a_spread[rows], "fp8")
    frac = float(np.mean(codes_got != ref.a_codes[rows]))
    assert frac <= 0.02, f"{frac:.4f} of the fp8 codes differ"


def check_a_mx(codes_packed, scales, ref, rows):
    """mxfp4 intermediate, element by element: block exponents inside the oracle's possible
    range and dequantised values within its spread.  Diagnostic as well: at most 1e-3 of the
    codes and of the block scales differ."""
    assert np.all((scales >= ref.q_lo[rows]) & (scales <= ref.q_hi[rows])), "block exponent outside its range"
    got_codes = oracle.fp4_unpack(codes_packed)
    got = oracle.mx_dequantize(got_codes, scales)
    want = oracle.mx_dequantize(ref.a_codes[rows], ref.a_scale[rows])
    _spread_check(got, want, ref.a_spread[rows], "mxfp4")
    assert (got_codes != ref.a_codes[rows]).mean() <= 1e-3, "codes differ beyond 1e-3"
    assert (scales != ref.a_scale[rows]).mean() <= 1e-3, "block scales differ beyond 1e-3"
