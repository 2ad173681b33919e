"""Routing: top-k gating (softmax or sigmoid score) and block-padded expert sorting.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
* "[Feat] Fuse TopKGatingSoftmax and MoE Sorting kernels" (ROCm/FlyDSL #582),
  "Motivation", "Relevant Files" and "Additional Details": a top-k gating
  softmax per token, followed by the MoE sorting step that groups the
  routed (token, slot) pairs by expert for the grouped GEMM.
* "[MoE] Port moe_gemm_2stage ... fp8" (ROCm/FlyDSL #947), the stage-2
  commit: a sorted id decodes to (token, slot) through a rank-3
  [tokens, topk, inter] view, and padding rows are sentinel rows that
  contribute nothing.
* "[Common] Optimize fused router forward/backward kernels"
  (NVIDIA/TransformerEngine #3012), "Changes / Forward kernels" and the
  flowchart: the score function (softmax or sigmoid) is applied and a top-k
  selection follows; "Hardening": topk must lie in [1, E] and
  tokens*experts must fit a signed 32-bit int.

Readings where the pages are silent (each also listed with the design notes):
* Selection compares the fp32 logits.  Softmax and sigmoid are strictly
  increasing, so this is exactly the top-k of the real-valued scores; it
  does not depend on how exp is rounded.  -0.0 equals +0.0.
* Ties go to the lower expert index; within a token the k picks are in
  descending score order (rank j = j-th best), so slot s = t*k + j.
* Weights are renormalised over the selected k (for softmax and sigmoid);
  with ``renorm=False`` they are the score itself at the selected experts.
* An expert with zero routed slots gets no block; each non-empty expert's
  list is padded up to a multiple of BLOCK_M with the sentinel T*k.
* ``num_valid`` is the total padded length; slots are stored flat
  (s = t*k + j); the tail of ``expert_ids`` past ``num_valid`` is -1.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

SCORES = ("softmax", "sigmoid")


def sorted_capacity(T: int, E: int, k: int, block_m: int) -> int:
    """Length that always holds the padded sorted list: each non-empty expert adds
    at most block_m-1 padding rows, and at most min(E, T*k) experts are non-empty."""
    n = T * k
    worst = n + min(E, n) * (block_m - 1)
    return -(-worst // block_m) * block_m


def select_topk(logits: np.ndarray, k: int) -> np.ndarray:
    """Per token, the k experts with the largest logits, best first, ties to the lower index.

    Step "top-k gating" of the fused routing kernel.  np.argsort with a stable
    sort on the negated logits orders each row by (logit descending, index
    ascending); the first k columns are the picks.
    """
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    if not (1 <= k <= E):
        raise ValueError("topk must lie in [1, E]")
    if np.isnan(logits).any():
        raise ValueError("NaN logits are outside the contract")
    neg = -logits.astype(np.float64)
    order = np.argsort(neg, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def _scores_f64(l: np.ndarray, score: str) -> np.ndarray:
    """Score of every expert: softmax over the token's E logits, or the sigmoid."""
    if score == "softmax":
        z = l - l.max(axis=1, keepdims=True)
        ez = np.exp(z)
        return ez / ez.sum(axis=1, keepdims=True)
    return 1.0 / (1.0 + np.exp(-l))


def _sigmoid_slope(l: np.ndarray) -> np.ndarray:
    """The sigmoid's derivative s (1 - s) = sigma(l) sigma(-l), float64."""
    with np.errstate(over="ignore"):
        return (1.0 / (1.0 + np.exp(-l))) * (1.0 / (1.0 + np.exp(l)))


def routing_weights_f64(logits: np.ndarray, ids: np.ndarray, score: str = "softmax",
                        renorm: bool = True) -> np.ndarray:
    """The routed weights in float64, unrounded (see routing_weights)."""
    if score not in SCORES:
        raise ValueError(f"score must be one of {SCORES}")
    l = np.asarray(logits, dtype=np.float64)
    sel = np.take_along_axis(_scores_f64(l, score), ids.astype(np.int64), axis=1)
    if renorm:
        sel = sel / sel.sum(axis=1, keepdims=True)
    return sel


def routing_weights(logits: np.ndarray, ids: np.ndarray, score: str = "softmax",
                    renorm: bool = True) -> np.ndarray:
    """Routed weights of the selected experts, float64 arithmetic, rounded once to fp32.

    softmax: p = softmax over all E experts of the token; sigmoid:
    p = 1 / (1 + exp(-logit)).  With renorm the selected p are divided by their
    sum, so each token's k weights sum to 1.
    """
    l = np.asarray(logits, dtype=np.float32).astype(np.float64)
    return routing_weights_f64(l, ids, score, renorm).astype(np.float32)


def routing_weights_backward(logits: np.ndarray, ids: np.ndarray, grad_w: np.ndarray,
                             score: str = "softmax", renorm: bool = True, magnitude: bool = False):
    """Gradient of the routed weights with respect to the logits, float64 [T, E].

    "[Common] Optimize fused router forward/backward kernels" (TransformerEngine #3012),
    "Changes / Backward kernels": the router's backward.  The pages give no formula;
    reading taken: the derivative of routing_weights at the selection the forward made
    (the selection is piecewise constant, so nothing flows through it).  Written as the
    Jacobian of w_j(l) contracted with grad_w, expert by expert:
    * softmax, renorm: w_j = e^{l_j} / sum_{i in S} e^{l_i}, dw_j/dl_m = w_j (d_jm - w_m), m in S;
    * sigmoid, renorm: w_j = s_j / sum_{i in S} s_i, dw_j/dl_m = s_m (1 - s_m) (d_jm - w_j) / sum s;
    * softmax over all E (no renorm): dw_j/dl_m = p_j (d_{e_j m} - p_m) for every expert m;
    * sigmoid (no renorm): dw_j/dl_m = s_j (1 - s_j) d_{e_j m}.
    With magnitude=True also returns, per element, the same contraction with every Jacobian
    entry's two parts (the Kronecker term and the coupling term) taken in absolute value and
    |grad_w|: the size of the terms a finite-precision evaluation adds up, against which its
    rounding is measured.
    """
    if score not in SCORES:
        raise ValueError(f"score must be one of {SCORES}")
    l = np.asarray(logits, dtype=np.float32).astype(np.float64)
    ids = np.asarray(ids, dtype=np.int64)
    g = np.asarray(grad_w, dtype=np.float64)
    T, E = l.shape
    k = ids.shape[1]
    p = _scores_f64(l, score)
    # sigmoid slope s (1 - s), written as sigma(l) sigma(-l): the same number without the
    # cancellation of 1 - s, which is exactly 0 in float64 for logits above about 37
    slope = _sigmoid_slope(l) if score == "sigmoid" else None
    out = np.zeros((T, E))
    mag = np.zeros((T, E))
    for t in range(T):
        sel = p[t, ids[t]]
        if renorm:
            w = sel / sel.sum()
            for j in range(k):
                for mi in range(k):
                    m = ids[t, mi]
                    d = 1.0 if mi == j else 0.0
                    if score == "softmax":
                        jac = w[j] * (d - w[mi])
                        size = w[j] * (d + w[mi])
                    else:
                        jac = slope[t, m] * (d - w[j]) / sel.sum()
                        size = slope[t, m] * (d + w[j]) / sel.sum()
                    out[t, m] += g[t, j] * jac
                    mag[t, m] += abs(g[t, j]) * size
        else:
            for j in range(k):
                e = ids[t, j]
                if score == "softmax":
                    out[t] += g[t, j] * p[t, e] * ((np.arange(E) == e) - p[t])
                    mag[t] += abs(g[t, j]) * p[t, e] * ((np.arange(E) == e) + p[t])
                else:
                    out[t, e] += g[t, j] * slope[t, e]
                    mag[t, e] += abs(g[t, j]) * slope[t, e]
    return (out, mag) if magnitude else out


def sort_slots(ids: np.ndarray, E: int, block_m: int, cap: int | None = None):
    """Block-padded expert sort of the flat slots s = t*k + j.

    Walk the slots in ascending order and append each to its expert's list;
    count c_e, pad each non-empty list up to a multiple of block_m with the
    sentinel T*k, and lay the lists out by expert index.  Returns
    (sorted_token_ids [cap], expert_ids [cap/block_m], num_valid).
    """
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    n = T * k
    if cap is None:
        cap = sorted_capacity(T, E, k, block_m)
    flat = ids.reshape(-1)
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert id out of range")
    lists = [[] for _ in range(E)]
    for s in range(n):
        lists[int(flat[s])].append(s)
    sentinel = n
    sorted_ids = np.full(cap, sentinel, dtype=np.int32)
    expert_ids = np.full(cap // block_m, -1, dtype=np.int32)
    offset = 0
    for e in range(E):
        c = len(lists[e])
        if c == 0:
            continue
        padded = -(-c // block_m) * block_m
        sorted_ids[offset:offset + c] = lists[e]
        expert_ids[offset // block_m:(offset + padded) // block_m] = e
        offset += padded
    if offset > cap:
        raise AssertionError("capacity bound violated")
    return sorted_ids, expert_ids, offset


@dataclass
class RouteResult:
    ids: np.ndarray            # int32 [T, k]
    weights: np.ndarray        # float32 [T, k]
    sorted_token_ids: np.ndarray  # int32 [cap]
    expert_ids: np.ndarray     # int32 [cap // block_m]
    num_valid: int
    cap: int


def route(logits: np.ndarray, k: int, block_m: int, score: str = "softmax",
          renorm: bool = True) -> RouteResult:
    """The whole routing step: select, weigh, sort."""
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    if T * E > 2**31 - 1:
        raise ValueError("tokens*experts must fit in int32")
    ids = select_topk(logits, k)
    w = routing_weights(logits, ids, score, renorm)
    cap = sorted_capacity(T, E, k, block_m)
    sids, eids, nv = sort_slots(ids, E, block_m, cap)
    return RouteResult(ids, w, sids, eids, nv, cap)


def group_scores(logits: np.ndarray, k: int, n_group: int, topk_group: int,
                 score: str = "softmax") -> np.ndarray:
    """Score of each expert group, float64 [T, n_group] (group-limited routing).

    "[Common] Optimize fused router forward/backward kernels" (TransformerEngine #3012),
    "Hardening" (topk must be a multiple of group_topk) and the review's note on the group
    scores of the forward kernels.  The pages give no formula; reading taken: the E experts
    form n_group groups of E/n_group consecutive experts, and a group's score is the sum of
    its m = k/topk_group largest expert scores (softmax over all E, or the sigmoid), added
    best first.
    """
    if score not in SCORES:
        raise ValueError(f"score must be one of {SCORES}")
    l = np.asarray(logits, dtype=np.float32).astype(np.float64)
    T, E = l.shape
    _check_groups(E, k, n_group, topk_group)
    m = k // topk_group
    p = _scores_f64(l, score)
    gs = np.zeros((T, n_group))
    size = E // n_group
    for t in range(T):
        for g in range(n_group):
            vals = p[t, g * size:(g + 1) * size]
            order = np.argsort(-vals, kind="stable")
            for r in range(m):
                gs[t, g] += vals[order[r]]
    return gs


def _check_groups(E: int, k: int, n_group: int, topk_group: int) -> None:
    if not (1 <= k <= E):
        raise ValueError("topk must lie in [1, E]")
    if n_group < 1 or E % n_group:
        raise ValueError("n_group must divide E")
    if not (1 <= topk_group <= n_group):
        raise ValueError("topk_group must lie in [1, n_group]")
    if k % topk_group:
        raise ValueError("topk must be a multiple of topk_group")
    if k > topk_group * (E // n_group):
        raise ValueError("the kept groups must hold at least topk experts")


def select_groups(gs: np.ndarray, topk_group: int) -> np.ndarray:
    """The topk_group groups with the largest scores per token, ties to the lower group
    index; bool [T, n_group]."""
    T, G = gs.shape
    order = np.argsort(-gs, axis=1, kind="stable")
    keep = np.zeros((T, G), dtype=bool)
    np.put_along_axis(keep, order[:, :topk_group], True, axis=1)
    return keep


def select_topk_grouped(logits: np.ndarray, k: int, n_group: int, topk_group: int,
                        score: str = "softmax") -> np.ndarray:
    """Group-limited top-k: the k best experts among the topk_group best groups.

    Reading (see group_scores): first the groups are ranked by their score and the best
    topk_group kept; the experts of the other groups are then excluded and the k largest
    logits among the rest are picked, best first, ties to the lower expert index.
    n_group = 1 (or topk_group = n_group) is the ungrouped select_topk.
    """
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    gs = group_scores(logits, k, n_group, topk_group, score)
    keep = select_groups(gs, topk_group)
    allowed = np.repeat(keep, E // n_group, axis=1)
    neg = np.where(allowed, -logits.astype(np.float64), np.inf)
    order = np.argsort(neg, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def route_grouped(logits: np.ndarray, k: int, block_m: int, n_group: int, topk_group: int,
                  score: str = "softmax", renorm: bool = True) -> RouteResult:
    """Routing with group-limited selection; weights and sort as in route()."""
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    if T * E > 2**31 - 1:
        raise ValueError("tokens*experts must fit in int32")
    ids = select_topk_grouped(logits, k, n_group, topk_group, score)
    w = routing_weights(logits, ids, score, renorm)
    cap = sorted_capacity(T, E, k, block_m)
    sids, eids, nv = sort_slots(ids, E, block_m, cap)
    return RouteResult(ids, w, sids, eids, nv, cap)


def aux_loss_scores(logits: np.ndarray, k: int, score: str = "softmax"):
    """Per-token expert scores and routing map for the load-balancing auxiliary loss.

    "[Common] Optimize fused router forward/backward kernels" (TransformerEngine #3012):
    the summary and the file table name a kernel computing the scores for the MoE
    auxiliary loss, forward and backward, benchmarked beside the top-k kernel.  The pages
    give no formula; reading taken: the balance loss averages a distribution over the
    experts per token and counts the tokens routed to each expert, so
    * scores [T, E] float64: softmax over all E; or the sigmoid divided by its sum over
      all E (a distribution as well);
    * routing map [T, E] bool: True at the token's top-k experts (select_topk).
    """
    l = np.asarray(logits, dtype=np.float32)
    T, E = l.shape
    ids = select_topk(l, k)
    rmap = np.zeros((T, E), dtype=bool)
    np.put_along_axis(rmap, ids.astype(np.int64), True, axis=1)
    return aux_loss_scores_f64(l.astype(np.float64), score), rmap


def aux_loss_scores_f64(logits: np.ndarray, score: str = "softmax") -> np.ndarray:
    """The scores of aux_loss_scores from float64 logits, unrounded."""
    if score not in SCORES:
        raise ValueError(f"score must be one of {SCORES}")
    s = _scores_f64(np.asarray(logits, dtype=np.float64), score)
    if score == "sigmoid":
        s = s / s.sum(axis=1, keepdims=True)
    return s


def aux_loss_scores_backward(logits: np.ndarray, grad_scores: np.ndarray,
                             score: str = "softmax", magnitude: bool = False):
    """Gradient of aux_loss_scores' scores with respect to the logits, float64 [T, E].

    Written as the Jacobian of the scores contracted with grad_scores, entry by entry:
    * softmax: dp_e/dl_c = p_e (d_ec - p_c);
    * normalised sigmoid, q_e = s_e / S with S = sum_i s_i:
      dq_e/dl_c = s_c (1 - s_c) (d_ec - q_e) / S.
    The routing map is piecewise constant and passes no gradient.  With magnitude=True also
    returns the contraction of |grad_scores| with the Jacobian whose two parts (Kronecker and
    coupling term) are taken in absolute value, as in routing_weights_backward.
    """
    if score not in SCORES:
        raise ValueError(f"score must be one of {SCORES}")
    l = np.asarray(logits, dtype=np.float32).astype(np.float64)
    g = np.asarray(grad_scores, dtype=np.float64)
    T, E = l.shape
    out = np.zeros((T, E))
    mag = np.zeros((T, E))
    eye = np.eye(E)
    for t in range(T):
        if score == "softmax":
            p = _scores_f64(l[t:t + 1], "softmax")[0]
            jac = p[:, None] * (eye - p[None, :])          # [e, c]
            size = p[:, None] * (eye + p[None, :])
        else:
            s = 1.0 / (1.0 + np.exp(-l[t]))
            S = s.sum()
            q = s / S
            slope = _sigmoid_slope(l[t])  # s (1 - s) without cancellation
            jac = (eye - q[:, None]) * slope[None, :] / S
            size = (eye + q[:, None]) * slope[None, :] / S
        out[t] = g[t] @ jac
        mag[t] = np.abs(g[t]) @ size
    return (out, mag) if magnitude else out
