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
                             score: str = "softmax", renorm: bool = True) -> np.ndarray:
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
    """
    if score not in SCORES:
        raise ValueError(f"score must be one of {SCORES}")
    l = np.asarray(logits, dtype=np.float32).astype(np.float64)
    ids = np.asarray(ids, dtype=np.int64)
    g = np.asarray(grad_w, dtype=np.float64)
    T, E = l.shape
    k = ids.shape[1]
    p = _scores_f64(l, score)
    out = np.zeros((T, E))
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
                    else:
                        jac = sel[mi] * (1.0 - sel[mi]) * (d - w[j]) / sel.sum()
                    out[t, m] += g[t, j] * jac
        else:
            for j in range(k):
                e = ids[t, j]
                if score == "softmax":
                    out[t] += g[t, j] * p[t, e] * ((np.arange(E) == e) - p[t])
                else:
                    out[t, e] += g[t, j] * sel[j] * (1.0 - sel[j])
    return out


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
