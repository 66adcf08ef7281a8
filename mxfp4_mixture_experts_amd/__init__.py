"""Python binding of the MI355X (gfx950) routed MXFP4 Mixture-of-Experts layer.

Argument marshalling only: every step of the layer runs in the HIP kernels of ``libmoe_mxfp4.so``
(built in-tree by ``mxfp4_mixture_experts_amd.build``). torch supplies device memory and the current
stream. There is no CPU fallback: if the library is missing, importing the entry points raises.

The calls mirror the C ABI of ``include/moe_mxfp4.h``:

    ids, w = route_topk(logits, k)                 # router top-k + renormalise
    grp = group_tokens(ids, E)                     # expert histogram, prefix scan, permutation
    out = mxfp4_ffn(x, weights, w, grp, ...)       # gate_up + SwiGLU, down, weighted combine
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_mxfp4.so")

MOE_OK = 0
SCORE_SOFTMAX = 0
SCORE_SIGMOID = 1
UNFUSED_GATE_UP = 1
FORCE_SMALL_M = 2
FORCE_LARGE_M = 4
STAGE_GATE_UP = 0
STAGE_DOWN = 1
STAGE_COMBINE = 2

_lib = None


class MoeError(RuntimeError):
    pass


class FfnPlan(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int) for name in (
        "small_m_max", "launch_small", "launch_large", "small_gateup_grid", "small_down_grid",
        "large_gateup_grid", "large_down_grid", "combine_grid", "n_launches")]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


def load_library(path: str | None = None):
    """Load libmoe_mxfp4.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise MoeError(f"{p} is missing: build it with `python -m mxfp4_mixture_experts_amd.build` "
                       "(there is no CPU fallback)")
    lib = ctypes.CDLL(p)
    V = ctypes.c_void_p
    i = ctypes.c_int
    lib.moe_abi_version.restype = i
    lib.moe_status_string.argtypes = [i]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_route_topk.argtypes = [V, i, i, i, i, i, V, V, V]
    lib.moe_route_topk.restype = i
    lib.moe_router_gemm_topk_workspace_size.argtypes = [i, i, i]
    lib.moe_router_gemm_topk_workspace_size.restype = ctypes.c_size_t
    lib.moe_router_gemm_topk.argtypes = [V, V, i, i, i, i, i, i, V, V, V, V, ctypes.c_size_t, V]
    lib.moe_router_gemm_topk.restype = i
    lib.moe_group_tokens.argtypes = [V, i, i, i, V, V, V, V, V, V, V]
    lib.moe_group_tokens.restype = i
    lib.moe_route_group.argtypes = [V, i, i, i, i, i, V, V, V, V, V, V, V, V, V]
    lib.moe_route_group.restype = i
    lib.moe_mxfp4_ffn_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.moe_mxfp4_ffn_workspace_size.restype = ctypes.c_size_t
    lib.moe_mxfp4_ffn.argtypes = [V, i, i, i, i, i, V, V, V, V, V, V, V, V, V, V, V, ctypes.c_float,
                                  i, V, V, ctypes.c_size_t, V]
    lib.moe_mxfp4_ffn.restype = i
    lib.moe_mxfp4_ffn_plan.argtypes = [i, i, i, i, i, i, ctypes.POINTER(FfnPlan)]
    lib.moe_mxfp4_ffn_plan.restype = i
    lib.moe_set_small_m_max.argtypes = [i]
    lib.moe_set_small_m_max.restype = i
    lib.moe_set_dense_down_cols.argtypes = [i]
    lib.moe_set_dense_down_cols.restype = i
    lib.moe_set_stage_events.argtypes = [i, V, V]
    lib.moe_set_stage_events.restype = i
    if path is None:
        _lib = lib
    return lib


def _check(status: int, what: str):
    if status != MOE_OK:
        msg = load_library().moe_status_string(status).decode()
        raise MoeError(f"{what} failed: {msg} ({status})")


def _ptr(t: torch.Tensor | None):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t: torch.Tensor, dtype, name: str):
    if not t.is_cuda:
        raise MoeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise MoeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise MoeError(f"{name} must be contiguous")
    return t


def abi_version() -> int:
    return load_library().moe_abi_version()


def ffn_plan(T: int, H: int, I: int, E: int, k: int, flags: int = 0) -> dict:
    plan = FfnPlan()
    _check(load_library().moe_mxfp4_ffn_plan(T, H, I, E, k, flags, ctypes.byref(plan)), "moe_mxfp4_ffn_plan")
    return plan.as_dict()


def set_dense_down_cols(cols: int) -> int:
    """Force the dense down GEMM's column tile (256 or 224; 0 restores the per-shape choice);
    returns the previous setting."""
    prev = load_library().moe_set_dense_down_cols(int(cols))
    if prev < 0:
        _check(prev, "moe_set_dense_down_cols")
    return prev


def set_small_m_max(v: int) -> int:
    """Override the launch-table threshold (-1 restores the token-count table); returns the
    previous setting."""
    prev = load_library().moe_set_small_m_max(int(v))
    if prev < -1:
        _check(prev, "moe_set_small_m_max")
    return prev


def set_stage_events(stage: int, start, stop):
    """Record HIP events around one stage of every later mxfp4_ffn call (None clears)."""
    s = ctypes.c_void_p(start.cuda_event) if start is not None else None
    e = ctypes.c_void_p(stop.cuda_event) if stop is not None else None
    _check(load_library().moe_set_stage_events(stage, s, e), "moe_set_stage_events")


def ffn_workspace_size(T: int, H: int, I: int, E: int, k: int, flags: int = 0) -> int:
    n = load_library().moe_mxfp4_ffn_workspace_size(T, H, I, E, k, flags)
    if n == 0 and T > 0:
        raise MoeError("invalid sizes for moe_mxfp4_ffn_workspace_size")
    return n


def route_topk(logits: torch.Tensor, k: int, score_fn: int = SCORE_SOFTMAX, renorm: bool = True,
               ids: torch.Tensor | None = None, weights: torch.Tensor | None = None, stream=None):
    _dev(logits, torch.float32, "logits")
    T, E = logits.shape
    if ids is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if weights is None:
        weights = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _check(load_library().moe_route_topk(_ptr(logits), T, E, k, score_fn, int(bool(renorm)),
                                         _ptr(ids), _ptr(weights), _stream(stream)), "moe_route_topk")
    return ids, weights


def router_gemm_topk_workspace_size(T: int, H: int, E: int) -> int:
    n = load_library().moe_router_gemm_topk_workspace_size(T, H, E)
    if n == 0:
        raise MoeError("invalid sizes for moe_router_gemm_topk_workspace_size")
    return n


def router_gemm_topk(x: torch.Tensor, w_router: torch.Tensor, k: int, score_fn: int = SCORE_SOFTMAX,
                     renorm: bool = True, want_logits: bool = True, workspace: torch.Tensor | None = None,
                     stream=None):
    """logits = x . w_router^T (bf16, fp32 accumulation) and their top-k; returns
    (topk_ids, topk_w, logits or None)."""
    _dev(x, torch.bfloat16, "x")
    _dev(w_router, torch.bfloat16, "w_router")
    T, H = x.shape
    E = w_router.shape[0]
    if w_router.shape[1] != H:
        raise MoeError("w_router must be [E, H] with the H of x")
    ids = torch.empty((T, k), dtype=torch.int32, device=x.device)
    weights = torch.empty((T, k), dtype=torch.float32, device=x.device)
    logits = torch.empty((T, E), dtype=torch.float32, device=x.device) if want_logits else None
    need = router_gemm_topk_workspace_size(T, H, E)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    _check(load_library().moe_router_gemm_topk(_ptr(x), _ptr(w_router), T, H, E, int(k), int(score_fn),
                                               int(bool(renorm)), _ptr(logits), _ptr(ids), _ptr(weights),
                                               _ptr(workspace), workspace.numel() * workspace.element_size(),
                                               _stream(stream)), "moe_router_gemm_topk")
    return ids, weights, logits


@dataclass
class Grouping:
    counts: torch.Tensor
    offsets: torch.Tensor
    sorted_pair: torch.Tensor
    pair_pos: torch.Tensor
    active: torch.Tensor
    n_active: torch.Tensor

    @staticmethod
    def empty(T: int, k: int, E: int, device) -> "Grouping":
        P = max(T * k, 1)
        z = lambda n: torch.empty(n, dtype=torch.int32, device=device)  # noqa: E731
        return Grouping(z(E), z(E + 1), z(P), z(P), z(E), z(1))


def group_tokens(ids: torch.Tensor, E: int, out: Grouping | None = None, stream=None) -> Grouping:
    _dev(ids, torch.int32, "topk_ids")
    T, k = ids.shape
    g = out if out is not None else Grouping.empty(T, k, E, ids.device)
    _check(load_library().moe_group_tokens(_ptr(ids), T, k, E, _ptr(g.counts), _ptr(g.offsets),
                                           _ptr(g.sorted_pair), _ptr(g.pair_pos), _ptr(g.active),
                                           _ptr(g.n_active), _stream(stream)), "moe_group_tokens")
    return g


def route_group(logits: torch.Tensor, k: int, score_fn: int = SCORE_SOFTMAX, renorm: bool = True,
                ids: torch.Tensor | None = None, weights: torch.Tensor | None = None,
                out: Grouping | None = None, stream=None):
    """route_topk then group_tokens in one call (one launch for small batches)."""
    _dev(logits, torch.float32, "logits")
    T, E = logits.shape
    if ids is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if weights is None:
        weights = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    g = out if out is not None else Grouping.empty(T, k, E, logits.device)
    _check(load_library().moe_route_group(_ptr(logits), T, E, k, score_fn, int(bool(renorm)), _ptr(ids),
                                          _ptr(weights), _ptr(g.counts), _ptr(g.offsets),
                                          _ptr(g.sorted_pair), _ptr(g.pair_pos), _ptr(g.active),
                                          _ptr(g.n_active), _stream(stream)), "moe_route_group")
    return ids, weights, g


@dataclass
class Mxfp4Weights:
    """Expert weights in the library's MXFP4 layout (device tensors, uint8)."""
    w13_q: torch.Tensor  # [E, 2I, H/2]
    w13_s: torch.Tensor  # [E, 2I, H/32]
    w2_q: torch.Tensor   # [E, H, I/2]
    w2_s: torch.Tensor   # [E, H, I/32]

    @property
    def E(self) -> int:
        return self.w13_q.shape[0]

    @property
    def I(self) -> int:
        return self.w13_q.shape[1] // 2

    @property
    def H(self) -> int:
        return self.w2_q.shape[1]

    def validate(self):
        E, I, H = self.E, self.I, self.H
        for t, name, shape in ((self.w13_q, "w13_q", (E, 2 * I, H // 2)),
                               (self.w13_s, "w13_s", (E, 2 * I, H // 32)),
                               (self.w2_q, "w2_q", (E, H, I // 2)),
                               (self.w2_s, "w2_s", (E, H, I // 32))):
            _dev(t, torch.uint8, name)
            if tuple(t.shape) != shape:
                raise MoeError(f"{name} has shape {tuple(t.shape)}, expected {shape}")


def mxfp4_ffn(x: torch.Tensor, w: Mxfp4Weights, topk_w: torch.Tensor, grp: Grouping,
              clamp_limit: float = 0.0, flags: int = 0, out: torch.Tensor | None = None,
              workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """x: bf16 [T, H] (torch.bfloat16 or its uint16/int16 bit pattern); returns bf16 [T, H]."""
    if not x.is_cuda or x.dim() != 2:
        raise MoeError("x must be a 2-D device tensor")
    T, H = x.shape
    k = topk_w.shape[1] if topk_w.dim() == 2 else 1
    E, I = w.E, w.I
    _dev(topk_w, torch.float32, "topk_w")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    need = ffn_workspace_size(T, H, I, E, k, flags)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _check(load_library().moe_mxfp4_ffn(
        _ptr(x), T, H, I, E, k, _ptr(w.w13_q), _ptr(w.w13_s), _ptr(w.w2_q), _ptr(w.w2_s),
        _ptr(topk_w), _ptr(grp.counts), _ptr(grp.offsets), _ptr(grp.sorted_pair), _ptr(grp.pair_pos),
        _ptr(grp.active), _ptr(grp.n_active), float(clamp_limit), int(flags), _ptr(out),
        _ptr(workspace), workspace.numel(), _stream(stream)), "moe_mxfp4_ffn")
    return out


class MoELayer:
    """One routed MXFP4 MoE layer with every buffer preallocated for up to ``max_tokens`` tokens.

    ``forward`` enqueues route + group (one call) -> ffn on the current stream and allocates nothing,
    so it can be captured into a HIP graph (torch.cuda.CUDAGraph).
    """

    def __init__(self, weights: Mxfp4Weights, k: int, max_tokens: int, score_fn: int = SCORE_SOFTMAX,
                 renorm: bool = True, clamp_limit: float = 0.0, flags: int = 0, device="cuda"):
        weights.validate()
        self.w = weights
        self.k = k
        self.T = max_tokens
        self.score_fn = score_fn
        self.renorm = renorm
        self.clamp = clamp_limit
        self.flags = flags
        E, H, I = weights.E, weights.H, weights.I
        self.ids = torch.empty((max_tokens, k), dtype=torch.int32, device=device)
        self.topk_w = torch.empty((max_tokens, k), dtype=torch.float32, device=device)
        self.grp = Grouping.empty(max_tokens, k, E, device)
        self.out = torch.empty((max_tokens, H), dtype=torch.bfloat16, device=device)
        ws = ffn_workspace_size(max_tokens, H, I, E, k, flags)
        self.workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=device)

    def forward(self, x: torch.Tensor, logits: torch.Tensor, weights: Mxfp4Weights | None = None,
                stream=None) -> torch.Tensor:
        T = x.shape[0]
        if T > self.T:
            raise MoeError(f"{T} tokens exceed the layer's capacity {self.T}")
        w = weights if weights is not None else self.w
        ids, tw = self.ids[:T], self.topk_w[:T]
        route_group(logits, self.k, self.score_fn, self.renorm, ids, tw, self.grp, stream)
        return mxfp4_ffn(x, w, tw, self.grp, self.clamp, self.flags, self.out[:T], self.workspace, stream)
