"""Pins of the oracle's group-limited top-k and auxiliary-loss scores.

Brute force over subsets, library softmax/sigmoid, a hand-worked example, finite
differences of the float64 forward, and invariants."""

import itertools

import numpy as np
import pytest
from scipy.special import expit, softmax

from oracle import (
    aux_loss_scores,
    aux_loss_scores_backward,
    aux_loss_scores_f64,
    group_scores,
    route,
    route_grouped,
    select_groups,
    select_topk,
    select_topk_grouped,
)


def lib_scores(l, score):
    l = np.asarray(l, dtype=np.float64)
    return softmax(l, axis=1) if score == "softmax" else expit(l)


# ---------------------------------------------------------------------------- group-limited top-k
@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
@pytest.mark.parametrize("E,k,G,TG", [(8, 4, 4, 2), (12, 2, 3, 1), (12, 6, 4, 3), (16, 8, 8, 4), (10, 3, 5, 3)])
def test_group_scores_brute_force(score, E, k, G, TG):
    # a group's score is the best sum over all m-subsets of its experts' library scores
    rng = np.random.default_rng(E + 7 * k + G)
    l = rng.standard_normal((4, E)).astype(np.float32)
    m = k // TG
    p = lib_scores(l, score)
    got = group_scores(l, k, G, TG, score)
    size = E // G
    for t in range(4):
        for g in range(G):
            best = max(sum(c) for c in itertools.combinations(p[t, g * size:(g + 1) * size], m))
            assert got[t, g] == pytest.approx(best, rel=1e-13)


@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
@pytest.mark.parametrize("E,k,G,TG", [(8, 4, 4, 2), (12, 2, 3, 1), (12, 6, 4, 3), (16, 8, 8, 4), (10, 3, 5, 3)])
def test_grouped_selection_brute_force(score, E, k, G, TG):
    # the kept groups maximise the summed group score over all topk_group-subsets; the picks
    # are Python's sorted() over (-logit, index) restricted to the kept groups' experts
    rng = np.random.default_rng(3 * E + k + 11 * G)
    l = rng.standard_normal((6, E)).astype(np.float32)
    gs = group_scores(l, k, G, TG, score)
    keep = select_groups(gs, TG)
    ids = select_topk_grouped(l, k, G, TG, score)
    size = E // G
    for t in range(6):
        best = max(itertools.combinations(range(G), TG), key=lambda c: sum(gs[t, i] for i in c))
        assert sorted(np.flatnonzero(keep[t])) == sorted(best)
        allowed = [e for e in range(E) if keep[t, e // size]]
        keyed = sorted((-float(l[t, e]), e) for e in allowed)
        assert list(ids[t]) == [e for _, e in keyed[:k]]


def test_grouped_hand_worked_example():
    # E=8 in 4 groups of 2, k=4, topk_group=2, so m=2: a group scores its two experts.
    l = np.array([[5.0, -3.0, 4.0, 4.0, 3.5, 3.4, 0.0, 0.0]], dtype=np.float32)
    # softmax: group sums are proportional to e^5+e^-3 = 148.46, 2e^4 = 109.20,
    # e^3.5+e^3.4 = 63.07, 2: groups 0 and 1 stay; expert 1 (logit -3) is picked ahead of
    # expert 4 (3.5), which the ungrouped top-4 would take.
    assert list(select_topk_grouped(l, 4, 4, 2, "softmax")[0]) == [0, 2, 3, 1]
    assert list(select_topk(l, 4)[0]) == [0, 2, 3, 4]
    # sigmoid: s(5)+s(-3) = 1.0407, 2s(4) = 1.9640, s(3.5)+s(3.4) = 1.9384, 2s(0) = 1:
    # groups 1 and 2 stay, and the best expert (0) is not picked at all.
    assert list(select_topk_grouped(l, 4, 4, 2, "sigmoid")[0]) == [2, 3, 4, 5]
    gs = group_scores(l, 4, 4, 2, "sigmoid")[0]
    assert gs == pytest.approx([1.0407, 1.9640, 1.9384, 1.0], abs=1e-4)


def test_grouped_special_cases():
    rng = np.random.default_rng(5)
    l = rng.standard_normal((7, 24)).astype(np.float32)
    for score in ("softmax", "sigmoid"):
        # one group, or every group kept: the ungrouped selection
        assert np.array_equal(select_topk_grouped(l, 6, 1, 1, score), select_topk(l, 6))
        assert np.array_equal(select_topk_grouped(l, 6, 6, 6, score), select_topk(l, 6))
        # m = 1 keeps the groups holding the topk_group largest group maxima
        ids = select_topk_grouped(l, 4, 6, 4, score)
        gmax = l.reshape(7, 6, 4).max(axis=2)
        for t in range(7):
            kept = set(np.argsort(-gmax[t], kind="stable")[:4])
            assert {e // 4 for e in ids[t]} <= kept
    # all-equal logits: groups 0..topk_group-1, then experts in index order
    z = np.zeros((2, 16), dtype=np.float32)
    assert np.array_equal(select_topk_grouped(z, 4, 8, 2, "softmax"), np.tile([0, 1, 2, 3], (2, 1)))
    # route_grouped shares weights and sort with route when grouping is a no-op
    a, b = route_grouped(l, 6, 8, 1, 1, "sigmoid", True), route(l, 6, 8, "sigmoid", True)
    assert np.array_equal(a.ids, b.ids) and np.array_equal(a.weights, b.weights)
    assert np.array_equal(a.sorted_token_ids, b.sorted_token_ids) and a.num_valid == b.num_valid


def test_grouped_host_checks():
    l = np.zeros((1, 12), dtype=np.float32)
    for k, G, TG in [(4, 5, 2), (4, 4, 3), (4, 4, 0), (4, 4, 5), (0, 4, 1), (13, 4, 1), (8, 6, 2)]:
        with pytest.raises(ValueError):
            select_topk_grouped(l, k, G, TG)


# ---------------------------------------------------------------------------- aux-loss scores
@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
@pytest.mark.parametrize("E,k", [(8, 2), (33, 5), (64, 8)])
def test_aux_scores_library_and_map(score, E, k):
    rng = np.random.default_rng(E + k)
    l = (3 * rng.standard_normal((5, E))).astype(np.float32)
    s, rmap = aux_loss_scores(l, k, score)
    ref = lib_scores(l, score)
    if score == "sigmoid":
        ref = ref / ref.sum(axis=1, keepdims=True)
    assert np.allclose(s, ref, rtol=1e-13, atol=0)
    assert np.allclose(s.sum(axis=1), 1.0, rtol=1e-14)
    for t in range(5):
        keyed = sorted((-float(v), e) for e, v in enumerate(l[t]))
        assert sorted(np.flatnonzero(rmap[t])) == sorted(e for _, e in keyed[:k])


def test_aux_scores_special_cases():
    z = np.zeros((2, 10), dtype=np.float32)
    for score in ("softmax", "sigmoid"):
        s, rmap = aux_loss_scores(z, 3, score)
        assert np.allclose(s, 0.1, rtol=1e-15)            # uniform distribution
        assert np.array_equal(np.flatnonzero(rmap[0]), [0, 1, 2])
    rng = np.random.default_rng(2)
    l = rng.standard_normal((3, 12)).astype(np.float32)
    # softmax is invariant to a shift of the row; the normalised sigmoid is not
    s0 = aux_loss_scores_f64(l, "softmax")
    assert np.allclose(aux_loss_scores_f64(l.astype(np.float64) + 3.0, "softmax"), s0, rtol=1e-13)
    q0 = aux_loss_scores_f64(l, "sigmoid")
    assert not np.allclose(aux_loss_scores_f64(l.astype(np.float64) + 3.0, "sigmoid"), q0)


@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
@pytest.mark.parametrize("E", [4, 9, 33])
def test_aux_backward_matches_finite_differences(score, E):
    rng = np.random.default_rng(E)
    T = 3
    l = rng.standard_normal((T, E)).astype(np.float32).astype(np.float64)
    g = rng.standard_normal((T, E))
    got = aux_loss_scores_backward(l, g, score)
    h = 1e-6
    fd = np.zeros((T, E))
    for c in range(E):
        lp, lm = l.copy(), l.copy()
        lp[:, c] += h
        lm[:, c] -= h
        fd[:, c] = ((aux_loss_scores_f64(lp, score) - aux_loss_scores_f64(lm, score)) * g).sum(axis=1) / (2 * h)
    assert np.allclose(got, fd, atol=1e-8, rtol=1e-6)


def test_aux_backward_special_cases():
    rng = np.random.default_rng(4)
    l = rng.standard_normal((4, 12))
    for score in ("softmax", "sigmoid"):
        # the scores sum to 1 per token: a gradient equal on every expert has no effect
        assert np.allclose(aux_loss_scores_backward(l, np.full((4, 12), 0.3), score), 0.0, atol=1e-15)
    # softmax is shift-invariant, so each token's gradient sums to zero
    gr = aux_loss_scores_backward(l, rng.standard_normal((4, 12)), "softmax")
    assert np.allclose(gr.sum(axis=1), 0.0, atol=1e-15)


def test_aux_backward_magnitude():
    """The magnitude output: closed form for softmax, p_c (|g_c| + sum_e p_e |g_e|), on a
    uniform row; |gradient| <= magnitude on random rows."""
    E = 5
    g = np.array([[1.0, -2.0, 0.5, 0.0, 3.0]])
    out, mag = aux_loss_scores_backward(np.zeros((1, E)), g, "softmax", magnitude=True)
    p = 1.0 / E
    assert np.allclose(mag[0], p * (np.abs(g[0]) + p * np.abs(g[0]).sum()), rtol=1e-14, atol=0)
    rng = np.random.default_rng(6)
    l = rng.standard_normal((4, 9))
    gr = rng.standard_normal((4, 9))
    for score in ("softmax", "sigmoid"):
        o, m_ = aux_loss_scores_backward(l, gr, score, magnitude=True)
        assert np.array_equal(o, aux_loss_scores_backward(l, gr, score))
        assert np.all(np.abs(o) <= m_ * (1 + 1e-12))
