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


def compare_out(out_gpu: torch.Tensor, ref_out: np.ndarray, rows, tol: float, cos_min: float | None):
    """max|err| <= tol * rms(ref) over the given rows (and cosine >= cos_min)."""
    got = out_gpu.detach().float().cpu().double().numpy()[rows]
    ref = ref_out[rows]
    assert np.isfinite(got).all()
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = float(np.abs(got - ref).max())
    cos = float((got * ref).sum() / (np.linalg.norm(got) * np.linalg.norm(ref) + 1e-300))
    assert err <= tol * rms, f"max|err| {err:.4g} > {tol} * rms {rms:.4g} (ratio {err / rms:.4g}); cos {cos:.6f}"
    if cos_min is not None:
        assert cos >= cos_min, f"cosine {cos:.7f} < {cos_min}"
    return err / rms, cos


def compare_out_bf16_atomic(out_gpu: torch.Tensor, ref_out: np.ndarray, ref_contrib: np.ndarray, rows,
                            k: int, tol: float):
    """Packed bf16 atomic accumulation: each of a token's k contributions is rounded to bf16
    and each of the k atomic adds rounds the running sum to bf16, so on top of the fp32
    modes' bound tol * rms(ref) an element may move by (k + 1) * 2^-9 * sum_j |c_j| (half a
    bf16 step per rounding, of a value at most sum_j |c_j|).  Returns the largest fraction
    of that allowance used."""
    got = out_gpu.detach().float().cpu().double().numpy()[rows]
    ref = ref_out[rows]
    assert np.isfinite(got).all()
    rms = float(np.sqrt(np.mean(ref * ref)))
    D = ref.shape[1]
    s_abs = np.abs(ref_contrib.reshape(-1, k, D)[rows]).sum(axis=1)
    allow = tol * rms + (k + 1) * 2.0 ** -9 * s_abs
    err = np.abs(got - ref)
    used = float((err / allow).max())
    i = np.unravel_index(np.argmax(err / allow), err.shape)
    assert used <= 1.0, (f"err {err[i]:.4g} > allowance {allow[i]:.4g} at {i} (ref {ref[i]:.5g}, "
                         f"sum|c| {s_abs[i]:.4g}, rms {rms:.4g})")
    return used


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |v| (normal range)."""
    _, e = np.frexp(np.maximum(np.abs(v), 2.0 ** -126))
    return np.ldexp(1.0, e - 8)


def check_a_bf16(got: np.ndarray, want: np.ndarray):
    """bf16 intermediate (diagnostic): fp32-vs-fp64 accumulation order moves an element by
    at most a couple of ulp (plus a sliver of the row scale where the sums cancel); at most
    1% of the elements may differ by more than one ulp."""
    d = np.abs(got - want)
    ulp = bf16_ulp(want)
    rms = np.sqrt(np.mean(want * want))
    frac = float(np.mean(d > ulp * 1.0001))
    assert frac <= 0.01, f"{frac:.4f} of the bf16 intermediate is more than 1 ulp off"
    bound = 2.0 * ulp + 1e-3 * rms
    i = np.unravel_index(np.argmax(d - bound), d.shape)
    assert np.all(d <= bound), f"intermediate diff {d[i]:.4g} at {i} (value {want[i]:.4g}, ulp {ulp[i]:.3g})"


def e4m3_step(v: np.ndarray) -> np.ndarray:
    """Spacing of e4m3 numbers at |v| (subnormal spacing 2^-9 below 2^-6)."""
    _, e = np.frexp(np.maximum(np.abs(v), 2.0 ** -6))
    return np.ldexp(1.0, e - 4)


def check_a_fp8(codes_got, scale_got, codes_want, scale_want):
    """fp8 intermediate (diagnostic): scales within 1% (the row amax may move by a bf16 ulp);
    each value (in units of its row scale, max 448) within one e4m3 step of the oracle's, plus
    0.05: the fp8 MFMA keeps about 7e-5 of the sum of |products| (measured on gfx950), which
    moves values that cancel to near zero by a few subnormal steps; at most 2% of the codes
    differ."""
    from oracle import e4m3_decode
    rel = np.abs(scale_got.astype(np.float64) / scale_want - 1.0)
    assert rel.max() <= 1e-2, f"a_scale rel diff {rel.max():.3g}"
    vg = e4m3_decode(codes_got)
    vw = e4m3_decode(codes_want)
    step = e4m3_step(np.maximum(np.abs(vg), np.abs(vw)))
    d = np.abs(vg - vw)
    assert np.all(d <= 1.02 * step + 0.05), f"fp8 values differ by {np.max(d / step):.3g} steps"
    frac = float(np.mean(codes_got != codes_want))
    assert frac <= 0.02, f"{frac:.4f} of the fp8 codes differ"
