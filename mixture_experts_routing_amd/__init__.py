"""MI355X (gfx950) MoE-layer forward hot path: thin Python binding of libmoe.so.

Every step of the path runs in the HIP kernels of ``libmoe.so``; this module
only marshals torch tensors (device memory) and the current HIP stream into
the C ABI declared in ``include/moe.h``.  The functions carry the same names
as the C entry points.  There is no fallback: if the library is missing,
importing the binding's entry points raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "MoeError",
    "load_library",
    "moe_sorted_capacity",
    "moe_route_workspace_bytes",
    "moe_gemm1_workspace_bytes",
    "moe_forward_workspace_layout",
    "moe_forward_workspace_bytes",
    "moe_strerror",
    "moe_topk_softmax_sort",
    "moe_gemm1_gateup",
    "moe_gemm2_down",
    "moe_finalize",
    "moe_topk_softmax_backward",
    "moe_topk_softmax_sort_grouped",
    "moe_aux_loss_scores",
    "moe_aux_loss_scores_backward",
    "moe_preshuffle_weights",
    "moe_forward",
    "moe_forward_noalloc",
    "moe_forward_noalloc_max_bytes",
    "SCORE",
    "DTYPE",
    "MODE",
    "WS_FIELDS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

SCORE = {"softmax": 0, "sigmoid": 1}
DTYPE = {"bf16": 0, "fp8": 1, "mxfp4": 2}
PRESHUFFLED = 0x100  # dtype flag: weights in fragment order (moe_preshuffle_weights)
MODE = {"atomic": 0, "reduce": 1, "atomic_bf16": 2, "reduce_bf16": 3}
WS_FIELDS = ("topk_weights", "topk_ids", "sorted_token_ids", "expert_ids", "num_valid",
             "route_scratch", "a", "a_scale", "gemm1_scratch", "y")

_lib = None


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {moe_strerror(status)} (status {status})")
        self.status = status


_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

_SIGS = {
    "moe_sorted_capacity": (_I64, [_I, _I, _I, _I]),
    "moe_route_workspace_bytes": (_I64, [_I, _I, _I, _I]),
    "moe_gemm1_workspace_bytes": (_I64, [_I, _I, _I, _I]),
    "moe_forward_workspace_layout": (_I64, [_I, _I, _I, _I, _I, _I, _I, _I, _P]),
    "moe_forward_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I, _I, _I]),
    "moe_strerror": (ctypes.c_char_p, [_I]),
    "moe_topk_softmax_sort": (_I, [_P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _I64, _P, _P, _P, _SZ, _P]),
    "moe_gemm1_gateup": (_I, [_I, _P, _P, _P, _P, _P, _P, _P, _I64, _I, _I, _I, _I, _I, _I, _P, _P, _P, _SZ, _P]),
    "moe_topk_softmax_backward": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P]),
    "moe_topk_softmax_sort_grouped": (_I, [_P, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _I64, _P, _P, _P,
                                           _SZ, _P]),
    "moe_aux_loss_scores": (_I, [_P, _I, _I, _I, _I, _P, _P, _P]),
    "moe_aux_loss_scores_backward": (_I, [_P, _P, _I, _I, _I, _P, _P]),
    "moe_preshuffle_weights": (_I, [_I, _P, _I64, _I, _P, _P]),
    "moe_preshuffle_scales": (_I, [_P, _I64, _I, _P, _P]),
    "moe_gemm2_down": (_I, [_I, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I, _I, _I, _I, _I, _I, _I, _P, _P]),
    "moe_finalize": (_I, [_I, _P, _I, _I, _I, _P, _P]),
    "moe_forward": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _SZ, _P, _P]),
    "moe_forward_noalloc": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P]),
    "moe_forward_noalloc_max_bytes": (_I64, []),
}


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads libmoe.so (built by mixture_experts_routing_amd.build); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m mixture_experts_routing_amd.build` "
                          "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def moe_strerror(status: int) -> str:
    return load_library().moe_strerror(status).decode()


def _check(status: int, where: str) -> int:
    if status < 0:
        raise MoeError(status, where)
    return status


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def moe_sorted_capacity(T: int, E: int, topk: int, block_m: int) -> int:
    return _check(load_library().moe_sorted_capacity(T, E, topk, block_m), "moe_sorted_capacity")


def moe_route_workspace_bytes(T: int, E: int, topk: int, block_m: int) -> int:
    return _check(load_library().moe_route_workspace_bytes(T, E, topk, block_m), "moe_route_workspace_bytes")


def moe_gemm1_workspace_bytes(dtype: str, T: int, topk: int, I: int) -> int:
    return _check(load_library().moe_gemm1_workspace_bytes(DTYPE[dtype], T, topk, I), "moe_gemm1_workspace_bytes")


def moe_forward_workspace_layout(dtype: str, mode: str, T: int, E: int, topk: int, D: int, I: int,
                                 block_m: int):
    """(total_bytes, {field: byte offset or None})."""
    offs = (ctypes.c_int64 * len(WS_FIELDS))()
    total = _check(load_library().moe_forward_workspace_layout(
        DTYPE[dtype], MODE[mode], T, E, topk, D, I, block_m, ctypes.cast(offs, ctypes.c_void_p)),
        "moe_forward_workspace_layout")
    return total, {f: (None if offs[i] < 0 else offs[i]) for i, f in enumerate(WS_FIELDS)}


def moe_forward_workspace_bytes(dtype: str, mode: str, T: int, E: int, topk: int, D: int, I: int,
                                block_m: int) -> int:
    """Total bytes of moe_forward's workspace; raises for invalid arguments (the C call returns 0)."""
    n = load_library().moe_forward_workspace_bytes(DTYPE[dtype], MODE[mode], T, E, topk, D, I, block_m)
    if n == 0:
        moe_forward_workspace_layout(dtype, mode, T, E, topk, D, I, block_m)  # raises with the status
    return n


def _route_buffers(logits, topk, block_m, out, workspace):
    T, E = logits.shape
    dev = logits.device
    cap = moe_sorted_capacity(T, E, topk, block_m)
    if out is None:
        out = {
            "topk_weights": torch.empty(T, topk, dtype=torch.float32, device=dev),
            "topk_ids": torch.empty(T, topk, dtype=torch.int32, device=dev),
            "sorted_token_ids": torch.empty(cap, dtype=torch.int32, device=dev),
            "expert_ids": torch.empty(cap // block_m, dtype=torch.int32, device=dev),
            "num_valid": torch.empty(1, dtype=torch.int32, device=dev),
        }
    if workspace is None:
        nbytes = moe_route_workspace_bytes(T, E, topk, block_m)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev) if nbytes else None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return out, workspace, ws_bytes


def moe_topk_softmax_sort(logits: torch.Tensor, topk: int, block_m: int, score: str = "softmax",
                          renorm: bool = True, out: dict | None = None, workspace=None, stream=None):
    """Routing outputs: dict(topk_weights, topk_ids, sorted_token_ids, expert_ids, num_valid)."""
    T, E = logits.shape
    out, workspace, ws_bytes = _route_buffers(logits, topk, block_m, out, workspace)
    _check(load_library().moe_topk_softmax_sort(
        _ptr(logits), T, E, topk, SCORE[score], int(renorm), block_m, _ptr(out["topk_weights"]),
        _ptr(out["topk_ids"]), _ptr(out["sorted_token_ids"]), out["sorted_token_ids"].numel(),
        _ptr(out["expert_ids"]), _ptr(out["num_valid"]), _ptr(workspace), ws_bytes, _stream(stream)),
        "moe_topk_softmax_sort")
    return out


def moe_topk_softmax_sort_grouped(logits: torch.Tensor, topk: int, n_group: int, topk_group: int,
                                  block_m: int, score: str = "softmax", renorm: bool = True,
                                  out: dict | None = None, workspace=None, stream=None):
    """Group-limited routing; outputs as moe_topk_softmax_sort."""
    T, E = logits.shape
    out, workspace, ws_bytes = _route_buffers(logits, topk, block_m, out, workspace)
    _check(load_library().moe_topk_softmax_sort_grouped(
        _ptr(logits), T, E, topk, n_group, topk_group, SCORE[score], int(renorm), block_m,
        _ptr(out["topk_weights"]), _ptr(out["topk_ids"]), _ptr(out["sorted_token_ids"]),
        out["sorted_token_ids"].numel(), _ptr(out["expert_ids"]), _ptr(out["num_valid"]),
        _ptr(workspace), ws_bytes, _stream(stream)), "moe_topk_softmax_sort_grouped")
    return out


def moe_aux_loss_scores(logits, topk: int, score: str = "softmax", scores=None, routing_map=None,
                        stream=None):
    """Auxiliary-loss scores fp32 [T, E] and routing map bool [T, E]."""
    T, E = logits.shape
    if scores is None:
        scores = torch.empty(T, E, dtype=torch.float32, device=logits.device)
    if routing_map is None:
        routing_map = torch.empty(T, E, dtype=torch.bool, device=logits.device)
    _check(load_library().moe_aux_loss_scores(
        _ptr(logits), T, E, topk, SCORE[score], _ptr(scores), _ptr(routing_map), _stream(stream)),
        "moe_aux_loss_scores")
    return scores, routing_map


def moe_aux_loss_scores_backward(logits, grad_scores, score: str = "softmax", grad_logits=None,
                                 stream=None):
    """Gradient of the auxiliary-loss scores with respect to the logits: fp32 [T, E]."""
    T, E = logits.shape
    if grad_logits is None:
        grad_logits = torch.empty(T, E, dtype=torch.float32, device=logits.device)
    _check(load_library().moe_aux_loss_scores_backward(
        _ptr(logits), _ptr(grad_scores), T, E, SCORE[score], _ptr(grad_logits), _stream(stream)),
        "moe_aux_loss_scores_backward")
    return grad_logits


def moe_topk_softmax_backward(logits, topk_ids, topk_weights, grad_topk_weights, score: str = "softmax",
                              renorm: bool = True, grad_logits=None, stream=None):
    """Gradient of the routed weights with respect to the logits: fp32 [T, E]."""
    T, E = logits.shape
    k = topk_ids.shape[1]
    if grad_logits is None:
        grad_logits = torch.empty(T, E, dtype=torch.float32, device=logits.device)
    _check(load_library().moe_topk_softmax_backward(
        _ptr(logits), _ptr(topk_ids), _ptr(topk_weights), _ptr(grad_topk_weights), T, E, k, SCORE[score],
        int(renorm), _ptr(grad_logits), _stream(stream)), "moe_topk_softmax_backward")
    return grad_logits


def moe_gemm1_gateup(dtype: str, x, w1, route: dict, topk: int, block_m: int, x_scale=None,
                     w1_scale=None, a=None, a_scale=None, workspace=None, stream=None, preshuffled: bool = False):
    """Stage 1: returns (a, a_scale); a is bf16 [T*k, I] (fp8: uint8 e4m3 codes + fp32 scales;
    mxfp4: packed uint8 [T*k, I/2] + E8M0 uint8 [T*k, I/32])."""
    T, D = x.shape
    E, twoI, _ = w1.shape
    I = twoI // 2
    if dtype == "mxfp4":
        D *= 2
    dev = x.device
    if a is None:
        shape = (T * topk, I // 2) if dtype == "mxfp4" else (T * topk, I)
        a = torch.empty(*shape, dtype=torch.bfloat16 if dtype == "bf16" else torch.uint8, device=dev)
    if dtype == "fp8" and a_scale is None:
        a_scale = torch.empty(T * topk, dtype=torch.float32, device=dev)
    if dtype == "mxfp4" and a_scale is None:
        a_scale = torch.empty(T * topk, I // 32, dtype=torch.uint8, device=dev)
    if workspace is None and dtype in ("fp8", "mxfp4"):
        workspace = torch.empty(max(moe_gemm1_workspace_bytes(dtype, T, topk, I), 1), dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    sid = route["sorted_token_ids"]
    _check(load_library().moe_gemm1_gateup(
        DTYPE[dtype] | (PRESHUFFLED if preshuffled else 0), _ptr(x), _ptr(x_scale), _ptr(w1), _ptr(w1_scale), _ptr(sid),
        _ptr(route["expert_ids"]), _ptr(route["num_valid"]), sid.numel(), T, E, topk, D, I, block_m,
        _ptr(a), _ptr(a_scale), _ptr(workspace), ws_bytes, _stream(stream)), "moe_gemm1_gateup")
    return a, a_scale


def moe_gemm2_down(dtype: str, a, w2, route: dict, T: int, topk: int, block_m: int, mode: str,
                   a_scale=None, w2_scale=None, y=None, stream=None, preshuffled: bool = False):
    """Stage 2: returns y (ATOMIC: fp32 [T, D] accumulated into; REDUCE: fp32 [T*k, D];
    ATOMIC_BF16: bf16 [T, D] accumulated into; REDUCE_BF16: bf16 [T*k, D])."""
    E, D, I = w2.shape
    if dtype == "mxfp4":
        I *= 2
    dev = a.device
    if y is None:
        rows = T if mode in ("atomic", "atomic_bf16") else T * topk
        y = torch.zeros(rows, D, dtype=torch.bfloat16 if mode.endswith("bf16") else torch.float32, device=dev)
    sid = route["sorted_token_ids"]
    _check(load_library().moe_gemm2_down(
        DTYPE[dtype] | (PRESHUFFLED if preshuffled else 0), _ptr(a), _ptr(a_scale), _ptr(w2), _ptr(w2_scale), _ptr(route["topk_weights"]),
        _ptr(sid), _ptr(route["expert_ids"]), _ptr(route["num_valid"]), sid.numel(), T, E, topk, D, I,
        block_m, MODE[mode], _ptr(y), _stream(stream)), "moe_gemm2_down")
    return y


def moe_finalize(mode: str, y, T: int, topk: int, D: int, out=None, stream=None):
    """Combine: bf16 out [T, D] from the fp32 accumulator, the fp32 or bf16 slot rows
    (ATOMIC_BF16: no-op)."""
    if out is None:
        out = torch.empty(T, D, dtype=torch.bfloat16, device=y.device)
    _check(load_library().moe_finalize(MODE[mode], _ptr(y), T, topk, D, _ptr(out), _stream(stream)),
           "moe_finalize")
    return out


def moe_forward(dtype: str, logits, x, w1, w2, topk: int, block_m: int, mode: str = "atomic",
                score: str = "softmax", renorm: bool = True, x_scale=None, w1_scale=None,
                w2_scale=None, workspace=None, out=None, stream=None, preshuffled: bool = False):
    """Whole layer; returns (out bf16 [T, D], workspace uint8, {field: view into workspace}).
    preshuffled: w1 and w2 come from moe_preshuffle_weights."""
    T, D = x.shape
    E, twoI, _ = w1.shape
    I = twoI // 2
    if dtype == "mxfp4":
        D *= 2
    total, offs = moe_forward_workspace_layout(dtype, mode, T, E, topk, D, I, block_m)
    dev = x.device
    if workspace is None:
        workspace = torch.empty(total, dtype=torch.uint8, device=dev)
    if out is None:
        out = torch.empty(T, D, dtype=torch.bfloat16, device=dev)
    _check(load_library().moe_forward(
        DTYPE[dtype] | (PRESHUFFLED if preshuffled else 0), SCORE[score], int(renorm), MODE[mode], _ptr(logits), _ptr(x), _ptr(x_scale),
        _ptr(w1), _ptr(w1_scale), _ptr(w2), _ptr(w2_scale), T, E, topk, D, I, block_m, _ptr(workspace),
        workspace.numel(), _ptr(out), _stream(stream)), "moe_forward")
    return out, workspace, offs


def moe_forward_noalloc(dtype: str, logits, x, w1, w2, topk: int, block_m: int, out, mode: str = "atomic",
                        score: str = "softmax", renorm: bool = True, x_scale=None, w1_scale=None,
                        w2_scale=None, stream=None, preshuffled: bool = False):
    """moe_forward without a workspace argument (the library's static per-device array);
    `out` bf16 [T, D] is the caller's.  Returns out."""
    T, D = x.shape
    E, twoI, _ = w1.shape
    I = twoI // 2
    if dtype == "mxfp4":
        D *= 2
    _check(load_library().moe_forward_noalloc(
        DTYPE[dtype] | (PRESHUFFLED if preshuffled else 0), SCORE[score], int(renorm), MODE[mode], _ptr(logits),
        _ptr(x), _ptr(x_scale), _ptr(w1), _ptr(w1_scale), _ptr(w2), _ptr(w2_scale), T, E, topk, D, I, block_m,
        _ptr(out), _stream(stream)), "moe_forward_noalloc")
    return out


def moe_forward_noalloc_max_bytes() -> int:
    return load_library().moe_forward_noalloc_max_bytes()


def moe_preshuffle_weights(dtype: str, w, out=None, stream=None):
    """Weights [E, N, row storage] (bf16, or uint8 for fp8 / packed mxfp4) into fragment order,
    same shape and dtype (scales are not touched; mxfp4 scales: moe_preshuffle_scales)."""
    rows = w.numel() // w.shape[-1]
    K = w.shape[-1] * 2 if dtype == "mxfp4" else w.shape[-1]
    if out is None:
        out = torch.empty_like(w)
    _check(load_library().moe_preshuffle_weights(DTYPE[dtype], _ptr(w), rows, K, _ptr(out), _stream(stream)),
           "moe_preshuffle_weights")
    return out


def moe_preshuffle_scales(s, out=None, stream=None):
    """mxfp4 E8M0 weight scales uint8 [E, N, K/32] into fragment order (same shape), for calls
    with preshuffled=True."""
    rows = s.numel() // s.shape[-1]
    K = s.shape[-1] * 32
    if out is None:
        out = torch.empty_like(s)
    _check(load_library().moe_preshuffle_scales(_ptr(s), rows, K, _ptr(out), _stream(stream)),
           "moe_preshuffle_scales")
    return out


def workspace_views(workspace, offs: dict, dtype: str, mode: str, T: int, E: int, topk: int, D: int,
                    I: int, block_m: int) -> dict:
    """Typed views of moe_forward's intermediates inside its workspace."""
    cap = moe_sorted_capacity(T, E, topk, block_m)
    n = T * topk

    def view(field, count, tdtype, shape):
        o = offs[field]
        if o is None:
            return None
        nbytes = count * torch.empty(0, dtype=tdtype).element_size()
        return workspace[o:o + nbytes].view(tdtype).view(*shape)

    v = {
        "topk_weights": view("topk_weights", n, torch.float32, (T, topk)),
        "topk_ids": view("topk_ids", n, torch.int32, (T, topk)),
        "sorted_token_ids": view("sorted_token_ids", cap, torch.int32, (cap,)),
        "expert_ids": view("expert_ids", cap // block_m, torch.int32, (cap // block_m,)),
        "num_valid": view("num_valid", 1, torch.int32, (1,)),
        "a": (view("a", n * I // 2, torch.uint8, (n, I // 2)) if dtype == "mxfp4" else
              view("a", n * I, torch.bfloat16 if dtype == "bf16" else torch.uint8, (n, I))),
        "a_scale": (view("a_scale", n * I // 32, torch.uint8, (n, I // 32)) if dtype == "mxfp4" else
                    view("a_scale", n, torch.float32, (n,))),
        "a_pre": view("gemm1_scratch", n * I, torch.bfloat16, (n, I)),
    }
    rows = T if mode == "atomic" else n
    v["y"] = view("y", rows * D, torch.bfloat16 if mode == "reduce_bf16" else torch.float32, (rows, D))
    return v
