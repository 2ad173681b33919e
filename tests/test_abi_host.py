"""C-ABI checks that need no GPU: exports, host helpers, and every validation error path.

All calls here fail validation (or are pure host helpers), so no HIP call is made.
"""

import ctypes
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

OK, EINVAL, ERANGE, ENOSPC, EUNSUP, ELAUNCH = 0, -1, -2, -3, -4, -5

GOOD = 0x10000  # a non-null, 16-byte aligned fake device address (never dereferenced)
BAD_ALIGN = 0x10004


@pytest.fixture(scope="module")
def lib():
    import mixture_experts_routing_amd as m
    return m.load_library()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("moe_topk_softmax_sort", "moe_gemm1_gateup", "moe_gemm2_down", "moe_forward"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), f"libmoe.so does not export {n}"


@pytest.mark.parametrize("T,E,k,B", [(1, 8, 2, 16), (4, 8, 2, 16), (16, 256, 8, 16), (16, 128, 4, 64),
                                     (4096, 128, 4, 64), (8192, 2304, 36, 32), (16384, 385, 9, 64),
                                     (0, 8, 2, 16), (3, 1, 1, 32), (1, 8160, 8160, 64)])
def test_sorted_capacity_matches_oracle(lib, T, E, k, B):
    assert lib.moe_sorted_capacity(T, E, k, B) == oracle.sorted_capacity(T, E, k, B)


def test_workspace_layout(lib):
    import mixture_experts_routing_amd as m
    for dtype in ("bf16", "fp8", "mxfp4"):
        for mode in ("atomic", "reduce", "atomic_bf16", "reduce_bf16"):
            for (T, E, k, D, I, B) in [(4, 8, 2, 128, 128, 16), (8192, 2304, 36, 128, 128, 32),
                                       (16, 256, 8, 7168, 2048, 16)]:
                total, offs = m.moe_forward_workspace_layout(dtype, mode, T, E, k, D, I, B)
                n, cap = T * k, oracle.sorted_capacity(T, E, k, B)
                sizes = {"topk_weights": 4 * n, "topk_ids": 4 * n, "sorted_token_ids": 4 * cap,
                         "expert_ids": 4 * cap // B, "num_valid": 4,
                         "route_scratch": m.moe_route_workspace_bytes(T, E, k, B),
                         "a": n * I * 2 if dtype == "bf16" else n * I if dtype == "fp8" else n * I // 2,
                         "a_scale": 4 * n if dtype == "fp8" else n * I // 32 if dtype == "mxfp4" else 0,
                         "gemm1_scratch": 2 * n * I if dtype in ("fp8", "mxfp4") else 0,
                         "y": (0 if mode == "atomic_bf16" else 4 * D * T if mode == "atomic" else
                               4 * D * n if mode == "reduce" else 2 * D * n)}
                spans = []
                for f, o in offs.items():
                    if sizes[f] == 0:
                        assert o is None
                        continue
                    assert o is not None and o % 256 == 0
                    spans.append((o, o + sizes[f]))
                spans.sort()
                for (a0, a1), (b0, _) in zip(spans, spans[1:]):
                    assert a1 <= b0
                assert spans[-1][1] <= total


def route_call(lib, T=4, E=8, k=2, score=0, renorm=1, B=16, cap=None, ptrs=None, ws=0, ws_bytes=0):
    if cap is None:
        cap = max(oracle.sorted_capacity(T, E, k, B), 0) if 1 <= k <= E and B in (16, 32, 64) else 1 << 20
    p = dict(logits=GOOD, w=GOOD, ids=GOOD, sorted=GOOD, eids=GOOD, nv=GOOD)
    p.update(ptrs or {})
    return lib.moe_topk_softmax_sort(p["logits"], T, E, k, score, renorm, B, p["w"], p["ids"],
                                     p["sorted"], cap, p["eids"], p["nv"], ws, ws_bytes, None)


def test_forward_workspace_bytes(lib):
    """moe_forward_workspace_bytes returns the layout's total, and 0 for invalid arguments."""
    import mixture_experts_routing_amd as m
    for dtype in ("bf16", "fp8", "mxfp4"):
        for mode in ("atomic", "reduce", "atomic_bf16", "reduce_bf16"):
            for (T, E, k, D, I, B) in [(4, 8, 2, 128, 128, 16), (8192, 2304, 36, 128, 128, 32),
                                       (16, 256, 8, 7168, 2048, 16), (0, 8, 2, 128, 128, 16)]:
                total, _ = m.moe_forward_workspace_layout(dtype, mode, T, E, k, D, I, B)
                got = lib.moe_forward_workspace_bytes(m.DTYPE[dtype], m.MODE[mode], T, E, k, D, I, B)
                assert got == total > 0
                assert m.moe_forward_workspace_bytes(dtype, mode, T, E, k, D, I, B) == total
    # invalid: bad dtype, bad mode, topk > E, D not a multiple of 64, block_m 8, T*k*D past int32
    for args in [(7, 0, 4, 8, 2, 128, 128, 16), (0, 9, 4, 8, 2, 128, 128, 16), (0, 0, 4, 8, 9, 128, 128, 16),
                 (0, 0, 4, 8, 2, 100, 128, 16), (0, 0, 4, 8, 2, 128, 128, 8),
                 (0, 0, 1 << 20, 8, 8, 1 << 10, 128, 16)]:
        assert lib.moe_forward_workspace_bytes(*args) == 0, args
    with pytest.raises(m.MoeError):
        m.moe_forward_workspace_bytes("bf16", "atomic", 4, 8, 9, 128, 128, 16)


def test_forward_noalloc_host_checks(lib):
    """moe_forward_noalloc: the static workspace size, and the errors returned before any HIP
    call (a workspace need beyond the array gives MOE_ENOSPC; bad arguments as moe_forward)."""
    import mixture_experts_routing_amd as m
    assert lib.moe_forward_noalloc_max_bytes() == m.moe_forward_noalloc_max_bytes() == 32 << 20
    P = GOOD

    def call(dtype=0, mode=0, T=4, E=8, k=2, D=128, I=128, B=16, out=P, score=0, renorm=1):
        return lib.moe_forward_noalloc(dtype, score, renorm, mode, P, P, P, P, P, P, P, T, E, k, D, I, B, out, None)

    # the GPT-OSS prefill shape in reduce mode needs ~290 MB: rejected before any HIP call
    assert m.moe_forward_workspace_bytes("bf16", "reduce", 4096, 128, 4, 2880, 2880, 64) > 32 << 20
    assert call(0, 1, 4096, 128, 4, 2880, 2880, 64) == ENOSPC
    assert call(mode=7) == EINVAL
    assert call(score=5) == EINVAL
    assert call(k=9) == EINVAL
    assert call(D=100) == EUNSUP
    assert call(out=BAD_ALIGN) == EINVAL
    assert call(out=0) == EINVAL
    assert call(T=0) == OK  # nothing to do


def test_route_validation(lib):
    assert route_call(lib, k=0) == EINVAL
    assert route_call(lib, k=9) == EINVAL
    assert route_call(lib, T=-1) == EINVAL
    assert route_call(lib, E=0, k=1) == EINVAL
    assert route_call(lib, E=8161, k=2) == EUNSUP
    assert route_call(lib, B=8) == EUNSUP
    assert route_call(lib, B=128) == EUNSUP
    assert route_call(lib, T=2**20, E=4096, k=2) == ERANGE  # T*E > INT_MAX
    assert route_call(lib, score=2) == EINVAL
    assert route_call(lib, renorm=2) == EINVAL
    assert route_call(lib, cap=oracle.sorted_capacity(4, 8, 2, 16) - 1) == ENOSPC
    for key in ("logits", "w", "ids", "sorted", "eids", "nv"):
        assert route_call(lib, ptrs={key: None}) == EINVAL
        assert route_call(lib, ptrs={key: BAD_ALIGN}) == EINVAL
    # multi-workgroup path needs a workspace
    need = lib.moe_route_workspace_bytes(1000, 256, 8, 16)
    assert need > 0
    assert route_call(lib, T=1000, E=256, k=8, ws=GOOD, ws_bytes=need - 1) == ENOSPC
    assert route_call(lib, T=1000, E=256, k=8, ws=None, ws_bytes=need) == EINVAL
    assert lib.moe_route_workspace_bytes(16, 256, 8, 16) == 0
    # the larger of the two multi-workgroup layouts: int32 counts with totals and offsets, or byte
    # counts in rows of 16 chunks (one chunk of 64 tokens, 3000 experts: 48000 bytes)
    assert lib.moe_route_workspace_bytes(64, 3000, 8, 16) == 48128
    assert lib.moe_route_workspace_bytes(8192, 512, 4, 32) == 128 * 512 * 4 + 2 * 2048 + 512


def gemm1_call(lib, dtype=0, T=4, E=8, k=2, D=128, I=64, B=16, cap=None, ptrs=None, ws_bytes=1 << 30):
    if cap is None:
        cap = oracle.sorted_capacity(T, E, k, B) if (1 <= k <= E and B in (16, 32, 64) and T >= 0) else 1 << 20
    p = dict(x=GOOD, xs=GOOD, w1=GOOD, w1s=GOOD, sid=GOOD, eid=GOOD, nv=GOOD, a=GOOD, as_=GOOD, ws=GOOD)
    p.update(ptrs or {})
    return lib.moe_gemm1_gateup(dtype, p["x"], p["xs"], p["w1"], p["w1s"], p["sid"], p["eid"], p["nv"],
                                cap, T, E, k, D, I, B, p["a"], p["as_"], p["ws"], ws_bytes, None)


def test_gemm1_validation(lib):
    assert gemm1_call(lib, dtype=3) == EINVAL
    # mxfp4 needs whole 128-element MFMA steps along D and I
    assert gemm1_call(lib, dtype=2, D=128, I=64) == EUNSUP
    assert gemm1_call(lib, dtype=2, D=192, I=128) == EUNSUP
    for key in ("xs", "w1s", "as_", "ws"):
        assert gemm1_call(lib, dtype=2, I=128, ptrs={key: None}) == EINVAL
    assert gemm1_call(lib, dtype=2, I=128, ws_bytes=4 * 2 * 128 * 2 - 1) == ENOSPC
    assert gemm1_call(lib, D=100) == EUNSUP
    assert gemm1_call(lib, I=96) == EUNSUP
    assert gemm1_call(lib, D=0) == EUNSUP
    assert gemm1_call(lib, k=3, E=2) == EINVAL
    assert gemm1_call(lib, B=48) == EUNSUP
    assert gemm1_call(lib, cap=oracle.sorted_capacity(4, 8, 2, 16) - 16) == ENOSPC
    for key in ("x", "w1", "sid", "eid", "nv", "a"):
        assert gemm1_call(lib, ptrs={key: None}) == EINVAL
        assert gemm1_call(lib, ptrs={key: BAD_ALIGN}) == EINVAL
    # fp8 needs the three scales and the workspace
    for key in ("xs", "w1s", "as_", "ws"):
        assert gemm1_call(lib, dtype=1, ptrs={key: None}) == EINVAL
    assert gemm1_call(lib, dtype=1, ws_bytes=4 * 2 * 64 * 2 - 1) == ENOSPC
    assert gemm1_call(lib, T=70000, E=8, k=2, D=16384) == ERANGE  # T*k*D > INT_MAX
    # the Kimi-K2.5 share (k=9, D=7168): T=33288 is the largest T with T*k*D < 2^31
    kimi = dict(dtype=1, E=385, k=9, D=7168, I=512, B=64)
    assert 33288 * 9 * 7168 < 2**31 <= 33289 * 9 * 7168
    assert gemm1_call(lib, T=33289, **kimi) == ERANGE


def gemm2_call(lib, dtype=0, mode=0, T=4, E=8, k=2, D=128, I=64, B=16, cap=None, ptrs=None):
    if cap is None:
        cap = oracle.sorted_capacity(T, E, k, B)
    p = dict(a=GOOD, as_=GOOD, w2=GOOD, w2s=GOOD, tw=GOOD, sid=GOOD, eid=GOOD, nv=GOOD, y=GOOD)
    p.update(ptrs or {})
    return lib.moe_gemm2_down(dtype, p["a"], p["as_"], p["w2"], p["w2s"], p["tw"], p["sid"], p["eid"],
                              p["nv"], cap, T, E, k, D, I, B, mode, p["y"], None)


def test_gemm2_validation(lib):
    assert gemm2_call(lib, mode=4) == EINVAL
    assert gemm2_call(lib, mode=-1) == EINVAL
    assert gemm2_call(lib, dtype=-1) == EINVAL
    assert gemm2_call(lib, D=64 + 32) == EUNSUP
    assert gemm2_call(lib, cap=1) == ENOSPC
    for key in ("a", "w2", "tw", "sid", "eid", "nv", "y"):
        assert gemm2_call(lib, ptrs={key: None}) == EINVAL
        assert gemm2_call(lib, ptrs={key: BAD_ALIGN}) == EINVAL
    for key in ("as_", "w2s"):
        assert gemm2_call(lib, dtype=1, ptrs={key: None}) == EINVAL


def test_finalize_and_forward_validation(lib):
    assert lib.moe_finalize(4, GOOD, 4, 2, 128, GOOD, None) == EINVAL
    assert lib.moe_finalize(3, GOOD, 4, 2, 100, GOOD, None) == EUNSUP
    assert lib.moe_finalize(3, None, 4, 2, 128, GOOD, None) == EINVAL
    # packed bf16 atomics write out in stage 2: nothing to combine, no pointer is used
    assert lib.moe_finalize(2, None, 4, 2, 128, None, None) == OK
    assert lib.moe_finalize(2, None, 4, 2, 100, None, None) == EUNSUP
    assert lib.moe_finalize(0, GOOD, 4, 2, 100, GOOD, None) == EUNSUP
    assert lib.moe_finalize(0, None, 4, 2, 128, GOOD, None) == EINVAL
    assert lib.moe_finalize(1, GOOD, 4, 2, 128, BAD_ALIGN, None) == EINVAL
    assert lib.moe_finalize(0, GOOD, -1, 2, 128, GOOD, None) == EINVAL
    total = lib.moe_forward_workspace_layout(0, 0, 4, 8, 2, 128, 64, 16, None)
    assert total > 0

    def fwd(dtype=0, score=0, renorm=1, mode=0, T=4, E=8, k=2, D=128, I=64, B=16, ws_bytes=total, **ptrs):
        p = dict(logits=GOOD, x=GOOD, xs=GOOD, w1=GOOD, w1s=GOOD, w2=GOOD, w2s=GOOD, ws=GOOD, out=GOOD)
        p.update(ptrs)
        return lib.moe_forward(dtype, score, renorm, mode, p["logits"], p["x"], p["xs"], p["w1"], p["w1s"],
                               p["w2"], p["w2s"], T, E, k, D, I, B, p["ws"], ws_bytes, p["out"], None)

    assert fwd(mode=5) == EINVAL
    assert fwd(score=3) == EINVAL
    assert fwd(ws_bytes=total - 1) == ENOSPC
    assert fwd(k=0) == EINVAL
    assert fwd(E=9000, k=2) == EUNSUP
    for key in ("logits", "x", "w1", "w2", "ws", "out"):
        assert fwd(**{key: None}) == EINVAL
    total8 = lib.moe_forward_workspace_layout(1, 0, 4, 8, 2, 128, 64, 16, None)
    for key in ("xs", "w1s", "w2s"):
        assert fwd(dtype=1, ws_bytes=total8, **{key: None}) == EINVAL


def test_route_backward_validation(lib):
    def call(T=4, E=8, k=2, score=0, renorm=1, **ptrs):
        p = dict(l=GOOD, ids=GOOD, w=GOOD, g=GOOD, out=GOOD)
        p.update(ptrs)
        return lib.moe_topk_softmax_backward(p["l"], p["ids"], p["w"], p["g"], T, E, k, score, renorm, p["out"], None)

    assert call(k=0) == EINVAL
    assert call(k=9) == EINVAL
    assert call(T=-1) == EINVAL
    assert call(E=9000, k=2) == EUNSUP
    assert call(score=2) == EINVAL
    assert call(renorm=2) == EINVAL
    assert call(T=300000, E=8000, k=2) == ERANGE
    assert call(T=0, l=None, out=None) == OK
    for key in ("l", "ids", "w", "g", "out"):
        assert call(**{key: None}) == EINVAL
        assert call(**{key: BAD_ALIGN}) == EINVAL


def test_grouped_route_validation(lib):
    def call(T=4, E=16, k=4, G=4, TG=2, score=0, renorm=1, B=16, **ptrs):
        cap = max(oracle.sorted_capacity(T, E, k, B), 16) if 1 <= k <= E else 1 << 20
        p = dict(logits=GOOD, w=GOOD, ids=GOOD, sorted=GOOD, eids=GOOD, nv=GOOD)
        p.update(ptrs)
        return lib.moe_topk_softmax_sort_grouped(p["logits"], T, E, k, G, TG, score, renorm, B, p["w"],
                                                 p["ids"], p["sorted"], cap, p["eids"], p["nv"], 0, 0, None)

    assert call(G=3) == EINVAL          # n_group does not divide E
    assert call(G=0) == EINVAL
    assert call(TG=0) == EINVAL
    assert call(TG=5) == EINVAL         # topk_group > n_group
    assert call(k=3, TG=2) == EINVAL    # topk not a multiple of topk_group
    assert call(k=6, G=8, TG=2) == EINVAL  # 2 kept groups of 2 experts hold fewer than 6
    assert call(E=256, k=8, G=128, TG=4) == EUNSUP  # more than 64 groups
    assert call(E=8000, k=8, G=8, TG=4) == EUNSUP   # group-limited needs E <= 4096
    # every group kept: the plain top-k, so E = 8000 passes (the null pointer stops the call)
    assert call(E=8000, k=8, G=8, TG=8, nv=None) == EINVAL
    assert call(k=0) == EINVAL
    assert call(score=2) == EINVAL
    for key in ("logits", "w", "ids", "sorted", "eids", "nv"):
        assert call(**{key: None}) == EINVAL


def test_aux_scores_validation(lib):
    def fwd(T=4, E=8, k=2, score=0, l=GOOD, s=GOOD, m=GOOD):
        return lib.moe_aux_loss_scores(l, T, E, k, score, s, m, None)

    def bwd(T=4, E=8, score=0, l=GOOD, g=GOOD, o=GOOD):
        return lib.moe_aux_loss_scores_backward(l, g, T, E, score, o, None)

    assert fwd(k=0) == EINVAL and fwd(k=9) == EINVAL and fwd(T=-1) == EINVAL
    assert fwd(E=5000, k=2) == EUNSUP and bwd(E=5000) == EUNSUP
    assert fwd(T=600000, E=4096) == ERANGE and bwd(T=600000, E=4096) == ERANGE
    assert fwd(score=2) == EINVAL and bwd(score=2) == EINVAL
    assert fwd(T=0, l=None, s=None, m=None) == OK and bwd(T=0, l=None, g=None, o=None) == OK
    for key in ("l", "s", "m"):
        assert fwd(**{key: None}) == EINVAL and fwd(**{key: BAD_ALIGN}) == EINVAL
    for key in ("l", "g", "o"):
        assert bwd(**{key: None}) == EINVAL and bwd(**{key: BAD_ALIGN}) == EINVAL


def test_preshuffle_validation(lib):
    PRE = 0x100

    def ps(dtype=0, rows=32, K=128, w=GOOD, o=0x20000):
        return lib.moe_preshuffle_weights(dtype, w, rows, K, o, None)

    assert ps(dtype=3) == EINVAL and ps(dtype=PRE) == EINVAL   # flags are not a dtype here
    assert ps(rows=-16) == EINVAL and ps(K=0) == EINVAL
    assert ps(rows=24) == EUNSUP                                  # not whole 16-row groups
    assert ps(dtype=0, K=96) == EUNSUP                            # bf16 rows of 192 bytes
    assert ps(dtype=1, K=192) == EUNSUP                           # fp8 rows of 192 bytes
    assert ps(dtype=2, K=384) == EUNSUP                           # mxfp4 rows of 192 bytes
    assert ps(rows=0, w=None, o=None) == OK
    assert ps(w=None) == EINVAL and ps(o=BAD_ALIGN) == EINVAL and ps(o=GOOD) == EINVAL  # w == out
    # the flag on the GEMM calls: fp8 rows must be whole 128-byte chunks (D = 192 is not)
    assert gemm1_call(lib, dtype=1 | PRE, D=192, I=128) == EUNSUP
    assert gemm2_call(lib, dtype=1 | PRE, D=128, I=192) == EUNSUP
    assert gemm1_call(lib, dtype=3 | PRE) == EINVAL
    # and is ignored by the workspace functions
    assert lib.moe_gemm1_workspace_bytes(1 | PRE, 4, 2, 128) == lib.moe_gemm1_workspace_bytes(1, 4, 2, 128)


def test_preshuffle_scales_validation(lib):
    def pss(rows=32, K=256, s=GOOD, o=0x20000):
        return lib.moe_preshuffle_scales(s, rows, K, o, None)

    assert pss(rows=-16) == EINVAL and pss(K=0) == EINVAL
    assert pss(rows=24) == EUNSUP                                 # not whole 16-row groups
    assert pss(K=128) == EUNSUP and pss(K=288) == EUNSUP          # not whole 256-element chunks
    assert pss(rows=0, s=None, o=None) == OK
    assert pss(s=None) == EINVAL and pss(o=None) == EINVAL
    assert pss(o=BAD_ALIGN) == EINVAL and pss(o=GOOD) == EINVAL   # s == out


def test_strerror(lib):
    import mixture_experts_routing_amd as m
    texts = {m.moe_strerror(s) for s in (OK, EINVAL, ERANGE, ENOSPC, EUNSUP, ELAUNCH)}
    assert len(texts) == 6
    assert "unknown" in m.moe_strerror(-99)


def test_missing_library_fails_loudly(tmp_path):
    import mixture_experts_routing_amd as m
    saved = m._lib
    m._lib = None
    try:
        with pytest.raises(ImportError):
            m.load_library(str(tmp_path / "nope.so"))
    finally:
        m._lib = saved
