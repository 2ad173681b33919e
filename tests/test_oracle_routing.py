"""Pins of the routing oracle: brute force, crafted ties, closed forms, library special cases, invariants."""

import math

import numpy as np
import pytest
import torch

from oracle import route, routing_weights, select_topk, sort_slots, sorted_capacity


def brute_topk(row, k):
    # independent of numpy: Python's sorted() over (-logit, index) tuples
    keyed = sorted((-float(v), e) for e, v in enumerate(row))
    return [e for _, e in keyed[:k]]


def brute_sort(ids, E, B):
    # independent of the oracle's bucket walk: scan expert by expert over all slots
    T, k = ids.shape
    out, eids = [], []
    for e in range(E):
        seg = [t * k + j for t in range(T) for j in range(k) if ids[t, j] == e]
        if not seg:
            continue
        pad = -(-len(seg) // B) * B
        out += seg + [T * k] * (pad - len(seg))
        eids += [e] * (pad // B)
    return out, eids


@pytest.mark.parametrize("seed", range(6))
def test_select_brute_force_random_and_tied(seed):
    rng = np.random.default_rng(seed)
    for T, E, k in [(5, 8, 2), (3, 16, 5), (4, 7, 7), (2, 33, 1)]:
        for gen in ("normal", "ties3", "dupcols", "zeros"):
            if gen == "normal":
                l = rng.standard_normal((T, E)).astype(np.float32)
            elif gen == "ties3":
                l = rng.integers(-1, 2, (T, E)).astype(np.float32)
            elif gen == "dupcols":
                l = rng.standard_normal((T, E)).astype(np.float32)
                l[:, E // 2:] = l[:, : E - E // 2]  # second half repeats the first
            else:
                l = rng.choice(np.array([0.0, -0.0, 1.0], dtype=np.float32), (T, E))
            ids = select_topk(l, k)
            for t in range(T):
                assert list(ids[t]) == brute_topk(l[t], k)


def test_all_equal_rows_pick_first_k():
    l = np.full((3, 10), 0.25, dtype=np.float32)
    assert np.array_equal(select_topk(l, 4), np.tile(np.arange(4), (3, 1)))
    l = np.zeros((1, 6), dtype=np.float32)
    l[0, ::2] = -0.0
    assert list(select_topk(l, 3)[0]) == [0, 1, 2]  # -0.0 ties with +0.0


def test_hand_worked_example():
    # T=3, E=4, k=2, BLOCK_M=4.
    l = np.array([[0.5, 2.0, -1.0, 2.0],      # tie 2.0 -> e1 before e3
                  [1.0, -0.0, 0.0, 3.0],      # e3 then e0
                  [-2.0, -2.0, -2.0, -2.0]],  # all equal -> e0, e1
                 dtype=np.float32)
    r = route(l, 2, 4)
    assert r.ids.tolist() == [[1, 3], [3, 0], [0, 1]]
    # slots: 0:(t0,e1) 1:(t0,e3) 2:(t1,e3) 3:(t1,e0) 4:(t2,e0) 5:(t2,e1); sentinel 6
    # e0:[3,4] e1:[0,5] e2:[] e3:[1,2]; each padded to 4; e2 gets no block
    assert r.cap == 20  # roundup(6 + min(4,6)*3, 4)
    assert r.num_valid == 12
    assert r.sorted_token_ids.tolist() == [3, 4, 6, 6, 0, 5, 6, 6, 1, 2, 6, 6] + [6] * 8
    assert r.expert_ids.tolist() == [0, 1, 3, -1, -1]
    # softmax renormalised over the pick = softmax of the picked logits
    w1 = 1.0 / (1.0 + math.exp(-2.0))
    assert r.weights[0].tolist() == [0.5, 0.5]
    assert r.weights[1].tolist() == [np.float32(w1), np.float32(1.0 - w1)]
    assert r.weights[2].tolist() == [0.5, 0.5]
    # sigmoid renormalised: sigma(3)/(sigma(3)+sigma(1))
    ws = routing_weights(l, r.ids, "sigmoid", True)
    s3, s1 = 1 / (1 + math.exp(-3.0)), 1 / (1 + math.exp(-1.0))
    assert ws[1].tolist() == [np.float32(s3 / (s3 + s1)), np.float32(s1 / (s3 + s1))]


def test_weights_closed_forms():
    rng = np.random.default_rng(3)
    l = rng.standard_normal((50, 12)).astype(np.float32)
    # k = 1 -> exactly 1.0 for both scores
    for score in ("softmax", "sigmoid"):
        ids = select_topk(l, 1)
        assert np.all(routing_weights(l, ids, score, True) == 1.0)
    # k = E with softmax -> the textbook softmax over all experts (torch, fp64), in pick order
    ids = select_topk(l, 12)
    w = routing_weights(l, ids, "softmax", True)
    ref = torch.softmax(torch.from_numpy(l).double(), dim=1).numpy()
    ref = np.take_along_axis(ref, ids.astype(np.int64), axis=1).astype(np.float32)
    assert np.array_equal(w, ref)
    # no renorm: the score itself at the picks
    ids = select_topk(l, 3)
    w = routing_weights(l, ids, "sigmoid", False)
    ref = torch.sigmoid(torch.from_numpy(l).double()).numpy()
    assert np.array_equal(w, np.take_along_axis(ref, ids.astype(np.int64), 1).astype(np.float32))
    w = routing_weights(l, ids, "softmax", False)
    ref = torch.softmax(torch.from_numpy(l).double(), dim=1).numpy()
    assert np.array_equal(w, np.take_along_axis(ref, ids.astype(np.int64), 1).astype(np.float32))
    # equal logits -> 1/k
    ids = select_topk(np.zeros((2, 9), np.float32), 4)
    assert np.all(routing_weights(np.zeros((2, 9), np.float32), ids) == np.float32(0.25))


@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
@pytest.mark.parametrize("E,k", [(8, 2), (256, 8), (512, 22), (2304, 36)])
def test_weights_sum_to_one_and_descend(score, E, k):
    l = np.random.default_rng(E + k).standard_normal((64, E)).astype(np.float32)
    ids = select_topk(l, k)
    w = routing_weights(l, ids, score, True).astype(np.float64)
    assert np.all(np.abs(w.sum(1) - 1.0) <= 1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)  # rank order is descending score


@pytest.mark.parametrize("seed", range(4))
def test_sort_brute_force_and_library(seed):
    rng = np.random.default_rng(seed)
    for T, E, k, B in [(4, 8, 2, 16), (16, 256, 8, 16), (37, 20, 5, 4), (1, 3, 3, 32), (64, 128, 4, 64)]:
        l = rng.standard_normal((T, E)).astype(np.float32)
        if seed == 1:  # skewed routing: a few hot experts
            l[:, :3] += 4.0
        ids = select_topk(l, k)
        cap = sorted_capacity(T, E, k, B)
        sids, eids, nv = sort_slots(ids, E, B, cap)
        bs, be = brute_sort(ids, E, B)
        assert nv == len(bs)
        assert sids[:nv].tolist() == bs
        assert np.all(sids[nv:] == T * k)
        assert eids[: nv // B].tolist() == be and np.all(eids[nv // B:] == -1)
        # library special case: a stable argsort of the flat ids is the unpadded order
        order = np.argsort(ids.reshape(-1), kind="stable")
        assert sids[sids < T * k].tolist() == order.tolist()


@pytest.mark.parametrize("T,E,k,B", [(16, 256, 8, 16), (4096, 128, 4, 64), (8192, 2304, 36, 32),
                                     (64, 385, 9, 64), (3, 8, 8, 16)])
def test_sort_invariants(T, E, k, B):
    l = np.random.default_rng(T).standard_normal((T, E)).astype(np.float32)
    r = route(l, k, B)
    sids, nv = r.sorted_token_ids, r.num_valid
    n = T * k
    valid = sids[:nv]
    real = valid[valid < n]
    assert sorted(real.tolist()) == list(range(n))        # each slot exactly once
    assert nv % B == 0 and nv <= r.cap == sorted_capacity(T, E, k, B)
    assert (valid == n).sum() == nv - n                    # #sentinels
    eids = r.expert_ids[: nv // B]
    assert np.all(np.diff(eids) >= 0)                      # experts in order
    flat = r.ids.reshape(-1)
    for b in range(nv // B):
        rows = valid[b * B:(b + 1) * B]
        rr = rows[rows < n]
        assert rr.size > 0                                 # no all-padding block
        assert np.all(flat[rr] == eids[b])                 # rows belong to the block's expert
        assert np.all(np.diff(rr) > 0)                     # ascending slots
        # padding only at the end of a block
        assert np.all(rows[: rr.size] < n)


def test_capacity_is_tight_when_every_expert_has_one_slot():
    # T*k = E distinct experts each with one slot: num_valid = E*B = capacity
    T, E, k, B = 4, 8, 2, 16
    l = np.zeros((T, E), np.float32)
    for t in range(T):
        l[t, 2 * t] = 2.0
        l[t, 2 * t + 1] = 1.0
    r = route(l, k, B)
    assert r.num_valid == E * B == r.cap


def test_host_checks():
    l = np.zeros((2, 4), np.float32)
    with pytest.raises(ValueError):
        select_topk(l, 0)
    with pytest.raises(ValueError):
        select_topk(l, 5)


# ---------------------------------------------------------------------------- backward
from oracle import routing_weights_backward, routing_weights_f64  # noqa: E402


@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
@pytest.mark.parametrize("renorm", [True, False])
@pytest.mark.parametrize("E,k", [(8, 2), (16, 5), (33, 1)])
def test_backward_matches_finite_differences(score, renorm, E, k):
    # central differences of the float64 forward at the fixed selection
    rng = np.random.default_rng(E * 10 + k)
    T = 3
    l = rng.standard_normal((T, E)).astype(np.float32).astype(np.float64)
    ids = select_topk(l.astype(np.float32), k)
    g = rng.standard_normal((T, k))
    got = routing_weights_backward(l, ids, g, score, renorm)
    h = 1e-6
    fd = np.zeros((T, E))
    for t in range(T):
        for m in range(E):
            lp, lm = l.copy(), l.copy()
            lp[t, m] += h
            lm[t, m] -= h
            dw = (routing_weights_f64(lp, ids, score, renorm) - routing_weights_f64(lm, ids, score, renorm)) / (2 * h)
            fd[t, m] = (dw[t] * g[t]).sum()
    assert np.allclose(got, fd, atol=1e-8, rtol=1e-6)


def test_backward_special_cases():
    rng = np.random.default_rng(3)
    l = rng.standard_normal((4, 12))
    ids = select_topk(l.astype(np.float32), 1)
    # one renormalised pick has weight 1 whatever the logits: zero gradient
    for score in ("softmax", "sigmoid"):
        assert not routing_weights_backward(l, ids, rng.standard_normal((4, 1)), score, True).any()
    # renormalised softmax is invariant to adding a constant to the picked logits, so each
    # token's gradient sums to zero; with a gradient equal on all picks it vanishes
    ids3 = select_topk(l.astype(np.float32), 3)
    gr = routing_weights_backward(l, ids3, rng.standard_normal((4, 3)), "softmax", True)
    assert np.allclose(gr.sum(axis=1), 0.0, atol=1e-15)
    assert np.allclose(routing_weights_backward(l, ids3, np.ones((4, 3)), "softmax", True), 0.0, atol=1e-15)
    # unpicked experts get no gradient except through the full softmax
    mask = np.zeros_like(l, dtype=bool)
    np.put_along_axis(mask, ids3, True, axis=1)
    for score, renorm in (("softmax", True), ("sigmoid", True), ("sigmoid", False)):
        assert not routing_weights_backward(l, ids3, np.ones((4, 3)) * 0.7, score, renorm)[~mask].any()


def test_backward_magnitude():
    """The magnitude output: a hand-worked case (two picks, softmax renormalised: weights 3/4
    and 1/4, gradient (1, -2)), and |gradient| <= magnitude on random data for every mode."""
    l = np.array([[0.0, np.log(3.0)]])
    ids = np.array([[1, 0]])
    out, mag = routing_weights_backward(l, ids, np.array([[1.0, -2.0]]), "softmax", True, magnitude=True)
    # (the logits pass through fp32, which moves ln 3 by about 1e-8)
    assert np.allclose(out[0], [-0.5625, 0.5625], atol=0, rtol=1e-7)
    assert np.allclose(mag[0], [0.8125, 1.6875], atol=0, rtol=1e-7)
    rng = np.random.default_rng(5)
    lr = rng.standard_normal((6, 20))
    ids4 = select_topk(lr.astype(np.float32), 4)
    gw = rng.standard_normal((6, 4))
    for score in ("softmax", "sigmoid"):
        for renorm in (True, False):
            o, m_ = routing_weights_backward(lr, ids4, gw, score, renorm, magnitude=True)
            assert np.array_equal(o, routing_weights_backward(lr, ids4, gw, score, renorm))
            assert np.all(np.abs(o) <= m_ * (1 + 1e-12) + 1e-300)
            assert np.all((m_ > 0) >= (o != 0))


def test_sigmoid_backward_large_logits():
    """The sigmoid's slope at large logits, where 1 - sigmoid(l) is 0 in float64: sigma(l)
    sigma(-l) = e^{-l} / (1 + e^{-l})^2 (about 4.25e-18 at l = 40, 0 only past exp's range)."""
    l = np.array([[40.0, -3.0, 90.0, 0.0]])
    ids = np.array([[2, 0]])
    out = routing_weights_backward(l, ids, np.array([[2.0, 0.5]]), "sigmoid", False)
    assert np.isclose(out[0, 0], 0.5 * np.exp(-40.0) / (1 + np.exp(-40.0)) ** 2, rtol=1e-14, atol=0)
    assert np.isclose(out[0, 2], 2.0 * np.exp(-90.0), rtol=1e-14, atol=0)
    assert out[0, 1] == 0 and out[0, 3] == 0
