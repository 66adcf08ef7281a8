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
SEPARATE_COMBINE = 8  # the combine as a launch of its own (never folded into down)
ACT_MXFP8 = 1  # W4A8: activations as MXFP8 (E4M3) blocks
ACT_MXFP4 = 2  # W4A4: activations as MXFP4 (E2M1) blocks
STAGE_GATE_UP = 0
STAGE_DOWN = 1
STAGE_COMBINE = 2

_lib = None


class MoeError(RuntimeError):
    pass


NUM_STAGES = 3


class FfnOptions(ctypes.Structure):
    """moe_ffn_options: per-call launch-table threshold, dense down column tile and stage events."""
    _fields_ = [("small_m_max", ctypes.c_int), ("dense_down_cols", ctypes.c_int),
                ("stage_start", ctypes.c_void_p * NUM_STAGES), ("stage_stop", ctypes.c_void_p * NUM_STAGES)]


def ffn_options(small_m_max: int = -1, dense_down_cols: int = 0, stage_events: dict | None = None) -> FfnOptions:
    """Options for one mxfp4_ffn call. stage_events maps a STAGE_* constant to a (start, stop) pair of
    torch.cuda.Event objects recorded around that stage on the call's stream."""
    o = FfnOptions()
    load_library().moe_ffn_options_init(ctypes.byref(o))
    o.small_m_max = int(small_m_max)
    o.dense_down_cols = int(dense_down_cols)
    for st, (a, b) in (stage_events or {}).items():
        o.stage_start[st] = a.cuda_event if a is not None else None
        o.stage_stop[st] = b.cuda_event if b is not None else None
    return o


class FfnPlan(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int) for name in (
        "small_m_max", "launch_small", "launch_large", "small_gateup_grid", "small_down_grid",
        "large_gateup_grid", "large_down_grid", "combine_grid", "n_launches", "fold_combine")]

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
    lib.moe_router_gemm_topk_ex.argtypes = [V, V, i, i, i, i, i, i, V, V, V, V, ctypes.c_size_t, i, V]
    lib.moe_router_gemm_topk_ex.restype = i
    lib.moe_layer_forward_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.moe_layer_forward_workspace_size.restype = ctypes.c_size_t
    lib.moe_layer_forward.argtypes = [V, V, i, i, i, i, i, i, i, V, V, V, V, ctypes.c_float, i, V, V, V, V, V,
                                      ctypes.c_size_t, V]
    lib.moe_layer_forward.restype = i
    lib.moe_layer_from_logits_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.moe_layer_from_logits_workspace_size.restype = ctypes.c_size_t
    lib.moe_layer_from_logits_routed.argtypes = [i, i, i, i, i, i, V]
    lib.moe_layer_from_logits_routed.restype = i
    lib.moe_layer_from_logits.argtypes = [V, V, i, i, i, i, i, i, i, V, V, V, V, ctypes.c_float, i, V, V, V, V,
                                          ctypes.c_size_t, V, V]
    lib.moe_layer_from_logits.restype = i
    lib.moe_group_tokens_workspace_size.argtypes = [i, i, i]
    lib.moe_group_tokens_workspace_size.restype = ctypes.c_size_t
    lib.moe_group_tokens.argtypes = [V, i, i, i, V, V, V, V, V, V, V, ctypes.c_size_t, V]
    lib.moe_group_tokens.restype = i
    lib.moe_route_group.argtypes = [V, i, i, i, i, i, V, V, V, V, V, V, V, V, V]
    lib.moe_route_group.restype = i
    lib.moe_mxfp4_ffn_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.moe_mxfp4_ffn_workspace_size.restype = ctypes.c_size_t
    lib.moe_mxfp4_ffn.argtypes = [V, i, i, i, i, i, V, V, V, V, V, V, V, V, V, V, V, ctypes.c_float,
                                  i, V, V, ctypes.c_size_t, V]
    lib.moe_mxfp4_ffn.restype = i
    lib.moe_mxfp4_ffn_ex.argtypes = [V, i, i, i, i, i, V, V, V, V, V, V, V, V, V, V, V, ctypes.c_float,
                                     i, V, V, ctypes.c_size_t, ctypes.POINTER(FfnOptions), V]
    lib.moe_mxfp4_ffn_ex.restype = i
    lib.moe_mxfp4_ffn_noalloc.argtypes = [V, i, i, i, i, i, V, V, V, V, V, V, V, V, V, V, V, ctypes.c_float,
                                          i, V, V]
    lib.moe_mxfp4_ffn_noalloc.restype = i
    lib.moe_mxfp4_ffn_noalloc_max_bytes.argtypes = []
    lib.moe_mxfp4_ffn_noalloc_max_bytes.restype = ctypes.c_size_t
    lib.moe_layer_decode_workspace_size.argtypes = [i, i, i, i, i]
    lib.moe_layer_decode_workspace_size.restype = ctypes.c_size_t
    lib.moe_layer_decode.argtypes = [V, V, i, i, i, i, i, i, i, V, V, V, V, ctypes.c_float, V, V, V, V,
                                     ctypes.c_size_t, V]
    lib.moe_layer_decode.restype = i
    lib.moe_mx_quantize.argtypes = [V, i, i, i, V, V, V]
    lib.moe_mx_quantize.restype = i
    lib.moe_mxfp4_ffn_mx_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.moe_mxfp4_ffn_mx_workspace_size.restype = ctypes.c_size_t
    lib.moe_mxfp4_ffn_mx.argtypes = [V, i, i, i, i, i, V, V, V, V, V, V, V, V, V, ctypes.c_float, i, V, V,
                                     ctypes.c_size_t, ctypes.POINTER(FfnOptions), V]
    lib.moe_mxfp4_ffn_mx.restype = i
    lib.moe_mxfp4_ffn_mx_h_offsets.argtypes = [i, i, i, i, i, i, ctypes.POINTER(ctypes.c_size_t),
                                               ctypes.POINTER(ctypes.c_size_t)]
    lib.moe_mxfp4_ffn_mx_h_offsets.restype = i
    lib.moe_ffn_options_init.argtypes = [ctypes.POINTER(FfnOptions)]
    lib.moe_ffn_options_init.restype = None
    lib.moe_mxfp4_ffn_plan.argtypes = [i, i, i, i, i, i, ctypes.POINTER(FfnOptions), ctypes.POINTER(FfnPlan)]
    lib.moe_mxfp4_ffn_plan.restype = i
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


def ffn_plan(T: int, H: int, I: int, E: int, k: int, flags: int = 0, options: FfnOptions | None = None) -> dict:
    plan = FfnPlan()
    _check(load_library().moe_mxfp4_ffn_plan(T, H, I, E, k, flags,
                                             ctypes.byref(options) if options is not None else None,
                                             ctypes.byref(plan)), "moe_mxfp4_ffn_plan")
    return plan.as_dict()


def ffn_workspace_size(T: int, H: int, I: int, E: int, k: int, flags: int = 0) -> int:
    n = load_library().moe_mxfp4_ffn_workspace_size(T, H, I, E, k, flags)
    if n == 0 and T > 0:
        raise MoeError("invalid sizes for moe_mxfp4_ffn_workspace_size")
    return n


def route_topk(logits: torch.Tensor, k: int, score_fn: int = SCORE_SOFTMAX, renorm: bool = True,
               ids: torch.Tensor | None = None, weights: torch.Tensor | None = None, stream=None):
    _dev(logits, torch.float32, "logits")
    if logits.dim() != 2:
        raise MoeError("logits must be [T, E]")
    T, E = logits.shape
    if ids is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if weights is None:
        weights = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    if ids.shape != (T, k) or weights.shape != (T, k):
        raise MoeError(f"ids and weights must be [{T}, {k}]")
    _dev(ids, torch.int32, "topk_ids")
    _dev(weights, torch.float32, "topk_w")
    _check(load_library().moe_route_topk(_ptr(logits), T, E, k, score_fn, int(bool(renorm)),
                                         _ptr(ids), _ptr(weights), _stream(stream)), "moe_route_topk")
    return ids, weights


def router_gemm_topk_workspace_size(T: int, H: int, E: int) -> int:
    n = load_library().moe_router_gemm_topk_workspace_size(T, H, E)
    if n == 0:
        raise MoeError("invalid sizes for moe_router_gemm_topk_workspace_size")
    return n


ROUTER_SPLIT_LAUNCH = 1


def router_workspace(T: int, H: int, E: int, device="cuda") -> torch.Tensor:
    """A zeroed workspace for router_gemm_topk (its first bytes are a counter that must start at 0)."""
    return torch.zeros(router_gemm_topk_workspace_size(T, H, E), dtype=torch.uint8, device=device)


def router_gemm_topk(x: torch.Tensor, w_router: torch.Tensor, k: int, score_fn: int = SCORE_SOFTMAX,
                     renorm: bool = True, want_logits: bool = True, workspace: torch.Tensor | None = None,
                     stream=None, split_launch: bool = False):
    """logits = x . w_router^T (bf16, fp32 accumulation) and their top-k; returns
    (topk_ids, topk_w, logits or None). `workspace` must come from router_workspace (zeroed once)."""
    _dev(x, torch.bfloat16, "x")
    _dev(w_router, torch.bfloat16, "w_router")
    T, H = x.shape
    E = w_router.shape[0]
    if w_router.shape[1] != H:
        raise MoeError("w_router must be [E, H] with the H of x")
    ids = torch.empty((T, k), dtype=torch.int32, device=x.device)
    weights = torch.empty((T, k), dtype=torch.float32, device=x.device)
    logits = torch.empty((T, E), dtype=torch.float32, device=x.device) if want_logits else None
    if workspace is None:
        workspace = router_workspace(T, H, E, x.device)
    _dev(workspace, torch.uint8, "workspace")
    _check(load_library().moe_router_gemm_topk_ex(_ptr(x), _ptr(w_router), T, H, E, int(k), int(score_fn),
                                                  int(bool(renorm)), _ptr(logits), _ptr(ids), _ptr(weights),
                                                  _ptr(workspace), workspace.numel(),
                                                  ROUTER_SPLIT_LAUNCH if split_launch else 0, _stream(stream)),
           "moe_router_gemm_topk_ex")
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

    def check(self, T: int, k: int, E: int):
        """Raise unless every buffer is a contiguous int32 device tensor large enough for T*k pairs
        over E experts."""
        P = T * k
        for name, need in (("counts", E), ("offsets", E + 1), ("sorted_pair", P), ("pair_pos", P),
                           ("active", E), ("n_active", 1)):
            t = _dev(getattr(self, name), torch.int32, f"grouping.{name}")
            if t.numel() < need:
                raise MoeError(f"grouping.{name} holds {t.numel()} entries, needs {need} "
                               f"(T={T}, k={k}, E={E})")


def group_workspace_size(T: int, k: int, E: int) -> int:
    n = load_library().moe_group_tokens_workspace_size(T, k, E)
    if n == ctypes.c_size_t(-1).value:
        raise MoeError("invalid sizes for moe_group_tokens_workspace_size")
    return n


def group_tokens(ids: torch.Tensor, E: int, out: Grouping | None = None, workspace: torch.Tensor | None = None,
                 stream=None) -> Grouping:
    _dev(ids, torch.int32, "topk_ids")
    if ids.dim() != 2:
        raise MoeError("topk_ids must be [T, k]")
    T, k = ids.shape
    g = out if out is not None else Grouping.empty(T, k, E, ids.device)
    g.check(T, k, E)
    need = group_workspace_size(T, k, E)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=ids.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load_library().moe_group_tokens(_ptr(ids), T, k, E, _ptr(g.counts), _ptr(g.offsets),
                                           _ptr(g.sorted_pair), _ptr(g.pair_pos), _ptr(g.active),
                                           _ptr(g.n_active), _ptr(workspace), ws_bytes, _stream(stream)),
           "moe_group_tokens")
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
    if ids.shape != (T, k) or weights.shape != (T, k):
        raise MoeError(f"ids and weights must be [{T}, {k}]")
    _dev(ids, torch.int32, "topk_ids")
    _dev(weights, torch.float32, "topk_w")
    g = out if out is not None else Grouping.empty(T, k, E, logits.device)
    g.check(T, k, E)
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


def _as_bf16(x: torch.Tensor, name: str = "x") -> torch.Tensor:
    """x as a contiguous 2-D bf16 device tensor (a uint16/int16 tensor of bf16 bit patterns is
    viewed as bf16)."""
    if not x.is_cuda or x.dim() != 2:
        raise MoeError(f"{name} must be a 2-D device tensor")
    if x.dtype in (torch.int16, torch.uint16):
        x = x.view(torch.bfloat16)
    return _dev(x, torch.bfloat16, name)


def ffn_check(x: torch.Tensor, w: Mxfp4Weights, topk_w: torch.Tensor, grp: Grouping,
              out: torch.Tensor | None = None, workspace: torch.Tensor | None = None, flags: int = 0):
    """Shape, dtype and size checks of one mxfp4_ffn call (host only, before any launch)."""
    x = _as_bf16(x)
    T, H = x.shape
    w.validate()
    if H != w.H:
        raise MoeError(f"x has hidden size {H}, the weights {w.H}")
    _dev(topk_w, torch.float32, "topk_w")
    if topk_w.dim() != 2 or topk_w.shape[0] != T:
        raise MoeError(f"topk_w must be [T={T}, k], got {tuple(topk_w.shape)}")
    k = topk_w.shape[1]
    grp.check(T, k, w.E)
    if out is not None:
        _dev(out, torch.bfloat16, "out")
        if tuple(out.shape) != (T, H):
            raise MoeError(f"out must be [{T}, {H}], got {tuple(out.shape)}")
    if workspace is not None:
        _dev(workspace, torch.uint8, "workspace")
        need = ffn_workspace_size(T, H, w.I, w.E, k, flags)
        if workspace.numel() < need:
            raise MoeError(f"workspace holds {workspace.numel()} bytes, needs {need}")
    return x, T, H, k


def mxfp4_ffn(x: torch.Tensor, w: Mxfp4Weights, topk_w: torch.Tensor, grp: Grouping,
              clamp_limit: float = 0.0, flags: int = 0, out: torch.Tensor | None = None,
              workspace: torch.Tensor | None = None, options: FfnOptions | None = None,
              stream=None) -> torch.Tensor:
    """x: bf16 [T, H] (torch.bfloat16 or its uint16/int16 bit pattern); returns bf16 [T, H]."""
    x, T, H, k = ffn_check(x, w, topk_w, grp, out, workspace, flags)
    E, I = w.E, w.I
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    need = ffn_workspace_size(T, H, I, E, k, flags)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _check(load_library().moe_mxfp4_ffn_ex(
        _ptr(x), T, H, I, E, k, _ptr(w.w13_q), _ptr(w.w13_s), _ptr(w.w2_q), _ptr(w.w2_s),
        _ptr(topk_w), _ptr(grp.counts), _ptr(grp.offsets), _ptr(grp.sorted_pair), _ptr(grp.pair_pos),
        _ptr(grp.active), _ptr(grp.n_active), float(clamp_limit), int(flags), _ptr(out),
        _ptr(workspace), workspace.numel(), ctypes.byref(options) if options is not None else None,
        _stream(stream)), "moe_mxfp4_ffn_ex")
    return out


def mxfp4_ffn_noalloc(x: torch.Tensor, w: Mxfp4Weights, topk_w: torch.Tensor, grp: Grouping,
                      clamp_limit: float = 0.0, flags: int = 0, out: torch.Tensor | None = None,
                      stream=None) -> torch.Tensor:
    """mxfp4_ffn without a workspace argument: the library uses its own fixed device scratch
    (moe_mxfp4_ffn_noalloc). Pass `out` to allocate nothing at all."""
    x, T, H, k = ffn_check(x, w, topk_w, grp, out, None, flags)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    _check(load_library().moe_mxfp4_ffn_noalloc(
        _ptr(x), T, H, w.I, w.E, k, _ptr(w.w13_q), _ptr(w.w13_s), _ptr(w.w2_q), _ptr(w.w2_s),
        _ptr(topk_w), _ptr(grp.counts), _ptr(grp.offsets), _ptr(grp.sorted_pair), _ptr(grp.pair_pos),
        _ptr(grp.active), _ptr(grp.n_active), float(clamp_limit), int(flags), _ptr(out), _stream(stream)),
        "moe_mxfp4_ffn_noalloc")
    return out


def mx_quantize(x: torch.Tensor, act_format: int = ACT_MXFP8, codes: torch.Tensor | None = None,
                scales: torch.Tensor | None = None, stream=None):
    """Quantise bf16 rows x [R, C] (C % 32 == 0) to MX blocks (moe_mx_quantize). Returns (codes u8
    [R, C] for MXFP8 or [R, C/2] for MXFP4, scale bytes u8 [R, C/32])."""
    x = _as_bf16(x)
    R, C = x.shape
    cw = C if act_format == ACT_MXFP8 else C // 2
    if codes is None:
        codes = torch.empty((R, cw), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((R, max(C // 32, 1)), dtype=torch.uint8, device=x.device)
    _dev(codes, torch.uint8, "codes")
    _dev(scales, torch.uint8, "scales")
    if tuple(codes.shape) != (R, cw) or tuple(scales.shape) != (R, C // 32):
        raise MoeError(f"codes must be [{R}, {cw}] and scales [{R}, {C // 32}]")
    _check(load_library().moe_mx_quantize(_ptr(x), R, C, int(act_format), _ptr(codes), _ptr(scales),
                                          _stream(stream)), "moe_mx_quantize")
    return codes, scales


def ffn_mx_workspace_size(T: int, H: int, I: int, E: int, k: int, act_format: int = ACT_MXFP8) -> int:
    n = load_library().moe_mxfp4_ffn_mx_workspace_size(T, H, I, E, k, int(act_format))
    if n == 0:
        raise MoeError(f"invalid sizes for moe_mxfp4_ffn_mx: T={T} H={H} I={I} E={E} k={k} act={act_format}")
    return n


def ffn_mx_h_view(workspace: torch.Tensor, T: int, H: int, I: int, E: int, k: int, act_format: int = ACT_MXFP8):
    """Views of the quantised h that moe_mxfp4_ffn_mx left in `workspace`: (codes u8 [T*k, I] or
    [T*k, I/2], scale bytes u8 [T*k, I/32]), rows in sorted order (moe_mxfp4_ffn_mx_h_offsets)."""
    co, so = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load_library().moe_mxfp4_ffn_mx_h_offsets(T, H, I, E, k, int(act_format), ctypes.byref(co),
                                                     ctypes.byref(so)), "moe_mxfp4_ffn_mx_h_offsets")
    P = T * k
    cw = I if act_format == ACT_MXFP8 else I // 2
    codes = workspace[co.value:co.value + P * cw].view(P, cw)
    scales = workspace[so.value:so.value + P * (I // 32)].view(P, I // 32)
    return codes, scales


def mxfp4_ffn_mx(x: torch.Tensor, w: Mxfp4Weights, topk_w: torch.Tensor, grp: Grouping,
                 clamp_limit: float = 0.0, act_format: int = ACT_MXFP8, out: torch.Tensor | None = None,
                 workspace: torch.Tensor | None = None, options: FfnOptions | None = None,
                 stream=None) -> torch.Tensor:
    """The expert FFN with MX-quantised activations (moe_mxfp4_ffn_mx): W4A8 for ACT_MXFP8, W4A4 for
    ACT_MXFP4. Returns bf16 [T, H]. With a `workspace`, ffn_mx_h_view shows the quantised h after the
    call. Of `options` only the stage events are used."""
    x, T, H, k = ffn_check(x, w, topk_w, grp, out, None, 0)
    E, I = w.E, w.I
    need = ffn_mx_workspace_size(T, H, I, E, k, act_format)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    _dev(workspace, torch.uint8, "workspace")
    if workspace.numel() < need:
        raise MoeError(f"workspace holds {workspace.numel()} bytes, needs {need}")
    _check(load_library().moe_mxfp4_ffn_mx(
        _ptr(x), T, H, I, E, k, _ptr(w.w13_q), _ptr(w.w13_s), _ptr(w.w2_q), _ptr(w.w2_s), _ptr(topk_w),
        _ptr(grp.counts), _ptr(grp.offsets), _ptr(grp.sorted_pair), _ptr(grp.pair_pos), float(clamp_limit),
        int(act_format), _ptr(out), _ptr(workspace), workspace.numel(),
        ctypes.byref(options) if options is not None else None, _stream(stream)), "moe_mxfp4_ffn_mx")
    return out


def layer_decode_workspace_size(T: int, H: int, I: int, E: int, k: int) -> int:
    """Bytes of workspace moe_layer_decode needs (0: the shape is not supported by the single launch)."""
    return load_library().moe_layer_decode_workspace_size(T, H, I, E, k)


def layer_decode_workspace(T: int, H: int, I: int, E: int, k: int, device="cuda") -> torch.Tensor:
    """A workspace for layer_decode, zeroed (its barrier counter must start at zero)."""
    n = layer_decode_workspace_size(T, H, I, E, k)
    if n == 0:
        raise MoeError(f"the single-launch layer does not support T={T} H={H} I={I} E={E} k={k}")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def layer_decode(logits: torch.Tensor, x: torch.Tensor, w: Mxfp4Weights, k: int, score_fn: int = SCORE_SOFTMAX,
                 renorm: bool = True, clamp_limit: float = 0.0, out: torch.Tensor | None = None,
                 workspace: torch.Tensor | None = None, ids: torch.Tensor | None = None,
                 weights: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """The whole layer in one launch (moe_layer_decode): logits f32 [T, E], x bf16 [T, H] -> bf16 [T, H].
    `workspace` must come from layer_decode_workspace (or be zeroed before its first use); `ids` and
    `weights` ([T, k]) receive the routing when given."""
    x = _as_bf16(x)
    T, H = x.shape
    w.validate()
    if H != w.H:
        raise MoeError(f"x has hidden size {H}, the weights {w.H}")
    _dev(logits, torch.float32, "logits")
    if tuple(logits.shape) != (T, w.E):
        raise MoeError(f"logits must be [{T}, {w.E}], got {tuple(logits.shape)}")
    for t, name, dt in ((ids, "topk_ids", torch.int32), (weights, "topk_w", torch.float32)):
        if t is not None:
            _dev(t, dt, name)
            if tuple(t.shape) != (T, k):
                raise MoeError(f"{name} must be [{T}, {k}]")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    else:
        _dev(out, torch.bfloat16, "out")
        if tuple(out.shape) != (T, H):
            raise MoeError(f"out must be [{T}, {H}]")
    if workspace is None:
        workspace = layer_decode_workspace(T, H, w.I, w.E, k, x.device)
    _dev(workspace, torch.uint8, "workspace")
    _check(load_library().moe_layer_decode(
        _ptr(logits), _ptr(x), T, H, w.I, w.E, int(k), int(score_fn), int(bool(renorm)), _ptr(w.w13_q),
        _ptr(w.w13_s), _ptr(w.w2_q), _ptr(w.w2_s), float(clamp_limit), _ptr(ids), _ptr(weights), _ptr(out),
        _ptr(workspace), workspace.numel(), _stream(stream)), "moe_layer_decode")
    return out


def layer_forward_workspace(T: int, H: int, I: int, E: int, k: int, flags: int = 0, device="cuda") -> torch.Tensor:
    """A zeroed workspace for layer_forward (its first bytes are the router's counter, which must start
    at 0)."""
    n = load_library().moe_layer_forward_workspace_size(T, H, I, E, k, flags)
    if n == 0:
        raise MoeError("invalid sizes for moe_layer_forward_workspace_size")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def layer_forward(x: torch.Tensor, w_router: torch.Tensor, w: Mxfp4Weights, k: int, score_fn: int = SCORE_SOFTMAX,
                  renorm: bool = True, clamp_limit: float = 0.0, flags: int = 0, out: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None, logits: torch.Tensor | None = None,
                  ids: torch.Tensor | None = None, weights: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """The whole layer from x (bf16 [T, H]) and the router weights (bf16 [E, H]): moe_layer_forward."""
    x = _as_bf16(x)
    T, H = x.shape
    w.validate()
    _dev(w_router, torch.bfloat16, "w_router")
    if tuple(w_router.shape) != (w.E, H) or H != w.H:
        raise MoeError(f"w_router must be [{w.E}, {w.H}] and x [T, {w.H}]")
    for t, name, dt, shape in ((logits, "logits", torch.float32, (T, w.E)), (ids, "topk_ids", torch.int32, (T, k)),
                               (weights, "topk_w", torch.float32, (T, k))):
        if t is not None:
            _dev(t, dt, name)
            if tuple(t.shape) != shape:
                raise MoeError(f"{name} must be {list(shape)}")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    elif tuple(out.shape) != (T, H):
        raise MoeError(f"out must be [{T}, {H}]")
    if workspace is None:
        workspace = layer_forward_workspace(T, H, w.I, w.E, k, flags, x.device)
    _dev(workspace, torch.uint8, "workspace")
    _check(load_library().moe_layer_forward(
        _ptr(x), _ptr(w_router), T, H, w.I, w.E, int(k), int(score_fn), int(bool(renorm)), _ptr(w.w13_q),
        _ptr(w.w13_s), _ptr(w.w2_q), _ptr(w.w2_s), float(clamp_limit), int(flags), _ptr(logits), _ptr(ids),
        _ptr(weights), _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream)), "moe_layer_forward")
    return out


def layer_from_logits_workspace(T: int, H: int, I: int, E: int, k: int, flags: int = 0, device="cuda") -> torch.Tensor:
    """A workspace for moe_layer_from_logits (no contents required)."""
    n = load_library().moe_layer_from_logits_workspace_size(T, H, I, E, k, flags)
    if n == 0:
        raise MoeError("invalid sizes for moe_layer_from_logits")
    return torch.empty(n, dtype=torch.uint8, device=device)


def layer_from_logits_routed(T: int, H: int, I: int, E: int, k: int, flags: int = 0,
                             options: FfnOptions | None = None) -> bool:
    """Whether moe_layer_from_logits routes and groups inside the gate_up launch for these sizes."""
    return bool(load_library().moe_layer_from_logits_routed(T, H, I, E, k, flags,
                                                            ctypes.byref(options) if options is not None else None))


def layer_from_logits(logits: torch.Tensor, x: torch.Tensor, w: Mxfp4Weights, k: int,
                      score_fn: int = SCORE_SOFTMAX, renorm: bool = True, clamp_limit: float = 0.0,
                      flags: int = 0, out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                      ids: torch.Tensor | None = None, weights: torch.Tensor | None = None,
                      options: FfnOptions | None = None, stream=None) -> torch.Tensor:
    """The whole layer from router logits (f32 [T, E]) and x (bf16 [T, H]): moe_layer_from_logits."""
    x = _as_bf16(x)
    T, H = x.shape
    w.validate()
    _dev(logits, torch.float32, "logits")
    if tuple(logits.shape) != (T, w.E) or H != w.H:
        raise MoeError(f"logits must be [{T}, {w.E}] and x [T, {w.H}]")
    for t, name, dt, shape in ((ids, "topk_ids", torch.int32, (T, k)), (weights, "topk_w", torch.float32, (T, k))):
        if t is not None:
            _dev(t, dt, name)
            if tuple(t.shape) != shape:
                raise MoeError(f"{name} must be {list(shape)}")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    elif tuple(out.shape) != (T, H):
        raise MoeError(f"out must be [{T}, {H}]")
    if workspace is None:
        workspace = layer_from_logits_workspace(T, H, w.I, w.E, k, flags, x.device)
    _dev(workspace, torch.uint8, "workspace")
    _check(load_library().moe_layer_from_logits(
        _ptr(logits), _ptr(x), T, H, w.I, w.E, int(k), int(score_fn), int(bool(renorm)), _ptr(w.w13_q),
        _ptr(w.w13_s), _ptr(w.w2_q), _ptr(w.w2_s), float(clamp_limit), int(flags), _ptr(ids), _ptr(weights),
        _ptr(out), _ptr(workspace), workspace.numel(), ctypes.byref(options) if options is not None else None,
        _stream(stream)), "moe_layer_from_logits")
    return out


class MoELayer:
    """One routed MXFP4 MoE layer with every buffer preallocated for up to ``max_tokens`` tokens.

    ``forward`` enqueues route + group (one call) -> ffn on the current stream and allocates nothing,
    so it can be captured into a HIP graph (torch.cuda.CUDAGraph).
    """

    def __init__(self, weights: Mxfp4Weights, k: int, max_tokens: int, score_fn: int = SCORE_SOFTMAX,
                 renorm: bool = True, clamp_limit: float = 0.0, flags: int = 0, device="cuda",
                 single_launch: bool = False, act_format: int = 0, from_logits: bool = False):
        """single_launch: run each forward as one moe_layer_decode launch (decode batches; every
        token count up to max_tokens must be supported by it). act_format ACT_MXFP8 / ACT_MXFP4: the
        FFN with MX-quantised activations (moe_mxfp4_ffn_mx; flags must be 0). from_logits: run each
        forward as one moe_layer_from_logits call (the routing inside the gate_up launch where it
        fits; the grouping then lives in the call's workspace and `grp` is not written)."""
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
        self.act_format = act_format
        if act_format and (flags or single_launch):
            raise MoeError("the activation-quantised FFN takes no flags and has no single-launch form")
        ws = (ffn_mx_workspace_size(max_tokens, H, I, E, k, act_format) if act_format
              else ffn_workspace_size(max_tokens, H, I, E, k, flags))
        self.workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=device)
        self.single_launch = single_launch
        self.from_logits = from_logits
        if from_logits:
            if single_launch or act_format:
                raise MoeError("from_logits excludes single_launch and act_format")
            self.lf_ws = layer_from_logits_workspace(max_tokens, H, I, E, k, flags, device)
        if single_launch:
            # sized for max_tokens, which bounds every smaller batch's need (zeroed once: the
            # barrier counter at its start must begin at zero)
            self.layer_ws = layer_decode_workspace(max_tokens, H, I, E, k, device)

    def forward(self, x: torch.Tensor, logits: torch.Tensor, weights: Mxfp4Weights | None = None,
                stream=None, options: FfnOptions | None = None) -> torch.Tensor:
        x = _as_bf16(x)
        T = x.shape[0]
        if T > self.T:
            raise MoeError(f"{T} tokens exceed the layer's capacity {self.T}")
        w = weights if weights is not None else self.w
        if (w.E, w.H, w.I) != (self.w.E, self.w.H, self.w.I):
            raise MoeError("weights differ in shape from the layer's")
        _dev(logits, torch.float32, "logits")
        if tuple(logits.shape) != (T, w.E):
            raise MoeError(f"logits must be [{T}, {w.E}], got {tuple(logits.shape)}")
        if x.shape[1] != w.H:
            raise MoeError(f"x has hidden size {x.shape[1]}, the layer {w.H}")
        ids, tw = self.ids[:T], self.topk_w[:T]
        if self.single_launch:
            return layer_decode(logits, x, w, self.k, self.score_fn, self.renorm, self.clamp, self.out[:T],
                                self.layer_ws, ids, tw, stream)
        if self.from_logits:
            return layer_from_logits(logits, x, w, self.k, self.score_fn, self.renorm, self.clamp, self.flags,
                                     self.out[:T], self.lf_ws, ids, tw, options, stream)
        route_group(logits, self.k, self.score_fn, self.renorm, ids, tw, self.grp, stream)
        if self.act_format:
            return mxfp4_ffn_mx(x, w, tw, self.grp, self.clamp, self.act_format, self.out[:T], self.workspace,
                                options, stream)
        return mxfp4_ffn(x, w, tw, self.grp, self.clamp, self.flags, self.out[:T], self.workspace, options,
                         stream)
