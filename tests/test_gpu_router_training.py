"""GPU parity of the group-limited router and the auxiliary-loss scores against the oracle.

Group-limited routing: ids, sort and expert ids bit-exact, weights rel <= 1e-6, as for the
plain router.  The group decisions come from fp64 sums of at most 36 terms on both sides,
which agree to about 1e-14 (relative); the test inputs are checked to hold no pair of groups
whose scores agree to within 1e-12 without being exactly equal, so every decision is unique.  Auxiliary-loss scores: routing map bit-exact,
scores rel <= 1e-6 (plus the smallest normal fp32, for underflow), backward element by element
|err| <= 1e-5 * the magnitude of the terms the element adds up."""

import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu_helpers import check_route

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    sys.stderr.write(f"\n[gpu] {request.node.nodeid}\n")
    sys.stderr.flush()
    yield


def _logits(T, E, gen, seed):
    if gen == "normal":
        return synth.logits(T, E, seed=seed)
    g = torch.Generator().manual_seed(seed)
    if gen == "ties3":
        return torch.randint(-1, 2, (T, E), generator=g).float()
    if gen == "equal":
        return torch.full((T, E), 0.5)
    if gen == "wide":
        return synth.logits(T, E, seed=seed) * 30.0
    raise ValueError(gen)


def _ambiguous_rows(l, k, G, TG, score):
    """Rows whose group decision fp64 rounding could flip: an oracle-kept and an oracle-dropped
    group whose scores agree to 1e-12 (relative), unless their m best logits are the same
    multiset (then both sides sum identical values and break the tie by group index)."""
    T, E = l.shape
    gs = oracle.group_scores(l, k, G, TG, score)
    keep = oracle.select_groups(gs, TG)
    size, m = E // G, k // TG
    amb = np.zeros(T, dtype=bool)
    for t in range(T):
        kept, dropped = np.flatnonzero(keep[t]), np.flatnonzero(~keep[t])
        if not len(dropped):
            continue
        for i in kept:
            close = dropped[np.abs(gs[t, dropped] - gs[t, i]) <= 1e-12 * abs(gs[t, i])]
            top_i = np.sort(l[t, i * size:(i + 1) * size])[-m:]
            for j in close:
                if not np.array_equal(top_i, np.sort(l[t, j * size:(j + 1) * size])[-m:]):
                    amb[t] = True
    return amb, gs


def _valid_grouped_pick(l_row, ids, gs_row, k, G, TG):
    """The picks are a correct group-limited top-k for some kept set that fp64 rounding allows."""
    E = len(l_row)
    size = E // G
    ids = [int(e) for e in ids]
    if len(set(ids)) != k or min(ids) < 0 or max(ids) >= E:
        return False
    thr = -np.sort(-gs_row)[TG - 1]
    tol = 1e-12 * abs(thr)
    groups = {e // size for e in ids}
    if len(groups) > TG or any(gs_row[g] < thr - tol for g in groups):
        return False
    keyed = [(-float(l_row[e]), e) for e in ids]
    if keyed != sorted(keyed):
        return False
    allowed = groups | {g for g in range(G) if gs_row[g] > thr + tol}
    last = keyed[-1]
    return all((-float(l_row[e]), e) > last for e in range(E) if e // size in allowed and e not in ids)


def run_grouped(logits, k, G, TG, B, score, renorm):
    import mixture_experts_routing_amd as m
    T, E = logits.shape
    cap = m.moe_sorted_capacity(T, E, k, B)
    dev = logits.device
    canary = -12345
    out = {
        "topk_weights": torch.full((T, k), float("nan"), device=dev),
        "topk_ids": torch.full((T, k), canary, dtype=torch.int32, device=dev),
        "sorted_token_ids": torch.full((cap,), canary, dtype=torch.int32, device=dev),
        "expert_ids": torch.full((cap // B,), canary, dtype=torch.int32, device=dev),
        "num_valid": torch.full((1,), canary, dtype=torch.int32, device=dev),
    }
    m.moe_topk_softmax_sort_grouped(logits, k, G, TG, B, score, renorm, out=out)
    torch.cuda.synchronize()
    return out


GROUPED = [
    # (T, E, k, n_group, topk_group, B, gen)
    (1, 256, 8, 8, 4, 16, "normal"), (16, 256, 8, 8, 4, 16, "normal"),      # one workgroup
    (100, 256, 8, 8, 4, 16, "normal"), (4096, 256, 8, 8, 4, 64, "normal"),  # two-launch, multi
    (37, 64, 6, 4, 3, 16, "normal"), (300, 384, 8, 8, 2, 32, "normal"),     # m = 2; groups of 48
    (200, 2304, 36, 36, 6, 32, "normal"),                                   # 36 groups, m = 6
    (16, 1024, 8, 16, 4, 16, "normal"),                                     # one workgroup, E = 1024
    (64, 512, 80, 8, 4, 32, "normal"),                                      # k > 64: exact path
    (50, 64, 4, 8, 2, 16, "ties3"), (20, 512, 8, 4, 2, 16, "equal"),        # exact ties
    (200, 256, 8, 8, 4, 16, "wide"),
    (16, 256, 8, 8, 1, 16, "normal"), (16, 256, 8, 256 // 4, 8, 16, "normal"),  # m = 8; 64 groups
]


@pytest.mark.parametrize("T,E,k,G,TG,B,gen", GROUPED)
@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
@pytest.mark.parametrize("renorm", [True, False])
def test_grouped_route(T, E, k, G, TG, B, gen, score, renorm):
    if not renorm and (T, E) not in ((16, 256), (4096, 256), (200, 2304), (64, 512)):
        pytest.skip("renorm=False on the DeepSeek shapes, 36 groups and the exact path")
    lg = _logits(T, E, gen, seed=T + E + k + G)
    l = lg.numpy()
    got = run_grouped(lg.cuda(), k, G, TG, B, score, renorm)
    ref = oracle.route_grouped(l, k, B, G, TG, score, renorm)
    amb, gs = _ambiguous_rows(l, k, G, TG, score)
    if amb.any():
        # rows fp64 rounding may decide either way: check the GPU's picks are valid, then hold
        # the rest of the outputs to the oracle's weights and sort of those picks
        # (saturated sigmoids of the wide logits put most groups at 2 - O(1e-15): every row)
        assert gen == "wide" or amb.mean() < 0.05, f"{amb.sum()} ambiguous rows"
        gids = got["topk_ids"].cpu().numpy()
        ids = ref.ids.copy()
        for t in np.flatnonzero(amb):
            assert _valid_grouped_pick(l[t], gids[t], gs[t], k, G, TG), f"row {t}: invalid picks {gids[t]}"
            ids[t] = gids[t]
        w = oracle.routing_weights(l, ids, score, renorm)
        sids, eids, nv = oracle.sort_slots(ids, E, B, ref.cap)
        ref = oracle.RouteResult(ids, w, sids, eids, nv, ref.cap)
    check_route(got, ref, T, k)


def test_grouped_route_reduces_to_plain_and_empty():
    import mixture_experts_routing_amd as m
    lg = synth.logits(300, 256, seed=5).cuda()
    a = m.moe_topk_softmax_sort_grouped(lg, 8, 8, 8, 16, "sigmoid", True)
    b = m.moe_topk_softmax_sort(lg, 8, 16, "sigmoid", True)
    torch.cuda.synchronize()
    for key in a:
        assert torch.equal(a[key], b[key]), key
    e = m.moe_topk_softmax_sort_grouped(torch.empty(0, 256, device="cuda"), 8, 8, 4, 16)
    torch.cuda.synchronize()
    assert int(e["num_valid"].item()) == 0


# ---------------------------------------------------------------------------- aux-loss scores
AUX = [
    # (T, E, k, gen)
    (4, 8, 2, "normal"), (33, 100, 5, "normal"), (64, 4096, 8, "normal"),
    (8192, 512, 22, "normal"), (8192, 2304, 36, "normal"),
    (16, 512, 80, "normal"), (40, 256, 8, "ties3"), (20, 130, 3, "equal"), (300, 512, 8, "wide"),
    (17, 700, 6, "normal"), (50, 1000, 10, "normal"),
]


def _rows(T):
    return np.arange(T) if T <= 300 else np.arange(0, T, 97)


@pytest.mark.parametrize("T,E,k,gen", AUX)
@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
def test_aux_scores(T, E, k, gen, score):
    import mixture_experts_routing_amd as m
    lg = _logits(T, E, gen, seed=T + E + k)
    s_ref, map_ref = oracle.aux_loss_scores(lg.numpy(), k, score)
    scores = torch.full((T, E), float("nan"), device="cuda")
    rmap = torch.full((T, E), True, dtype=torch.bool, device="cuda")
    m.moe_aux_loss_scores(lg.cuda(), k, score, scores=scores, routing_map=rmap)
    torch.cuda.synchronize()
    got_map = rmap.cpu().numpy()
    bad = np.argwhere(got_map != map_ref)
    assert bad.size == 0, f"routing map differs at {bad[:5].tolist()}"
    got = scores.cpu().double().numpy()
    excess = np.abs(got - s_ref) - (1e-6 * np.abs(s_ref) + 2.0 ** -126)
    rel = np.abs(got - s_ref) / np.maximum(np.abs(s_ref), 1e-38)
    assert excess.max() <= 0, f"scores rel err {rel.max():.3g} at {np.unravel_index(rel.argmax(), rel.shape)}"


@pytest.mark.parametrize("T,E,k,gen", [a for a in AUX if a[2] <= 36])
@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
def test_aux_scores_backward(T, E, k, gen, score):
    import mixture_experts_routing_amd as m
    lg = _logits(T, E, gen, seed=T + E)
    g = torch.randn(T, E, generator=torch.Generator().manual_seed(E), dtype=torch.float32)
    out = torch.full((T, E), float("nan"), device="cuda")
    m.moe_aux_loss_scores_backward(lg.cuda(), g.cuda(), score, grad_logits=out)
    torch.cuda.synchronize()
    rows = _rows(T)
    ref, mag = oracle.aux_loss_scores_backward(lg.numpy()[rows], g.numpy()[rows], score, magnitude=True)
    got = out.cpu().double().numpy()[rows]
    # element by element, against the magnitude of the terms each element adds up
    err = np.abs(got - ref)
    allow = 1e-5 * mag + 1e-30
    i = np.unravel_index(np.argmax(err / allow), err.shape)
    assert np.all(err <= allow), f"err {err[i]:.3g} > {allow[i]:.3g} at {i} (ref {ref[i]:.4g})"
