"""Plain CPU oracle for the routed MXFP4 MoE feed-forward — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import this
package. The product path (``mxfp4_mixture_experts_amd``) never imports it, and this package imports
nothing from the product path: the two share no code. The arithmetic lives in ``moe_oracle.c`` (plain
C, fp64); this module only builds it with gcc and marshals numpy arrays through ctypes.

Steps and their sources (page title, then section or element):
  * route   — "MTP1 Post-Portfolio Eager-Cycle Profile", Post-Portfolio Device Attribution table,
              native router select/normalize row;
  * group   — same table, direct M=2 route remap row;
  * ffn     — same table, compact routed MXFP4 GEMM and routed clamp-SwiGLU rows; the MXFP4 element
              format is the OCP Microscaling Formats (MX) v1.0 MXFP4 definition;
  * combine — the routing-weighted sum of each token's k expert outputs;
  * activation quantisation (the W4A8 / W4A4 mode) — the OCP Microscaling Formats (MX) v1.0
              specification: the MXFP8 (E4M3) and MXFP4 (E2M1) element formats and its shared-scale
              computation for a block of 32 values.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None

SCORE_SOFTMAX = 0
SCORE_SIGMOID = 1

ACT_NONE = 0
ACT_MXFP8 = 1
ACT_MXFP4 = 2


def compile_oracle(src: str, out: str) -> str:
    """Compile one oracle source with gcc (IEEE fp64: no fast-math, no FMA contraction)."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-I", _HERE, "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Build ``libmoe_oracle.so`` next to its source."""
    if force or not os.path.exists(_LIB_PATH):
        compile_oracle(_SRC, _LIB_PATH)
    return _LIB_PATH


class OracleLib:
    """ctypes bindings of one compiled oracle library (the default build, or a test's own build)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i = ctypes.c_int
        lib.oracle_e2m1_value.argtypes = [i]
        lib.oracle_e2m1_value.restype = ctypes.c_double
        lib.oracle_e8m0_value.argtypes = [i]
        lib.oracle_e8m0_value.restype = ctypes.c_double
        lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_double.restype = ctypes.c_double
        lib.oracle_double_to_bf16.argtypes = [ctypes.c_double]
        lib.oracle_double_to_bf16.restype = ctypes.c_uint16
        lib.oracle_mxfp4_element.argtypes = [P, P, i, ctypes.c_long, ctypes.c_long]
        lib.oracle_mxfp4_element.restype = ctypes.c_double
        lib.oracle_route_topk.argtypes = [P, i, i, i, i, i, P, P]
        lib.oracle_route_topk.restype = i
        lib.oracle_group_tokens.argtypes = [P, i, i, i, P, P, P, P, P, P]
        lib.oracle_group_tokens.restype = i
        lib.oracle_mxfp4_ffn.argtypes = [P, i, i, i, i, i, P, P, P, P, P, P, ctypes.c_double, i,
                                         P, P, P]
        lib.oracle_mxfp4_ffn.restype = i
        lib.oracle_mxfp4_ffn_act.argtypes = [P, i, i, i, i, i, P, P, P, P, P, P, ctypes.c_double, i,
                                             i, P, P, P, P]
        lib.oracle_mxfp4_ffn_act.restype = i
        lib.oracle_e4m3_value.argtypes = [i]
        lib.oracle_e4m3_value.restype = ctypes.c_double
        lib.oracle_e4m3_encode.argtypes = [ctypes.c_double]
        lib.oracle_e4m3_encode.restype = i
        lib.oracle_e2m1_encode.argtypes = [ctypes.c_double]
        lib.oracle_e2m1_encode.restype = i
        lib.oracle_mx_element.argtypes = [i, i]
        lib.oracle_mx_element.restype = ctypes.c_double
        lib.oracle_mx_quantize_block.argtypes = [P, i, P]
        lib.oracle_mx_quantize_block.restype = i
        lib.oracle_router_logits.argtypes = [P, P, i, i, i, i, P]
        lib.oracle_router_logits.restype = i
        lib.oracle_num_threads.argtypes = [i]
        lib.oracle_num_threads.restype = i
        self.lib = lib
        self.path = path

    def e2m1_value(self, code: int) -> float:
        return self.lib.oracle_e2m1_value(int(code))

    def e8m0_value(self, byte: int) -> float:
        return self.lib.oracle_e8m0_value(int(byte))

    def bf16_to_float(self, bits: int) -> float:
        return self.lib.oracle_bf16_to_double(int(bits))

    def float_to_bf16(self, v: float) -> int:
        return int(self.lib.oracle_double_to_bf16(float(v)))

    def mxfp4_element(self, q: np.ndarray, s: np.ndarray, K: int, n: int, kk: int) -> float:
        """Element (n, kk) of one expert's packed [N, K/2] codes and [N, K/32] scales."""
        q = _c(q, np.uint8)
        s = _c(s, np.uint8)
        return self.lib.oracle_mxfp4_element(_ptr(q), _ptr(s), int(K), int(n), int(kk))

    def e4m3_value(self, code: int) -> float:
        return self.lib.oracle_e4m3_value(int(code))

    def e4m3_encode(self, v: float) -> int:
        return int(self.lib.oracle_e4m3_encode(float(v)))

    def e2m1_encode(self, v: float) -> int:
        return int(self.lib.oracle_e2m1_encode(float(v)))

    def mx_element(self, fmt: int, code: int) -> float:
        return self.lib.oracle_mx_element(int(fmt), int(code))

    def mx_quantize_block(self, v, fmt: int):
        """Quantise 32 values to an MX block: returns (E8M0 scale byte, uint8[32] element codes)."""
        v = _c(v, np.float64)
        assert v.shape == (32,)
        codes = np.zeros(32, np.uint8)
        s = self.lib.oracle_mx_quantize_block(_ptr(v), int(fmt), _ptr(codes))
        return int(s), codes

    def mx_dequantize(self, v, fmt: int) -> np.ndarray:
        """Each consecutive 32-value block of v (float64, last axis a multiple of 32) quantised and
        decoded back, through mx_quantize_block."""
        v = _c(v, np.float64)
        flat = v.reshape(-1, 32)
        out = np.empty_like(flat)
        for b in range(flat.shape[0]):
            s, codes = self.mx_quantize_block(flat[b], fmt)
            out[b] = [self.mx_element(fmt, c) * self.e8m0_value(s) for c in codes]
        return out.reshape(v.shape)

    def route_topk(self, logits: np.ndarray, k: int, score_fn: int = SCORE_SOFTMAX,
                   renorm: bool = True):
        """Return (topk_ids int32[T,k], topk_w float64[T,k])."""
        logits = _c(logits, np.float32)
        T, E = logits.shape
        ids = np.zeros((T, k), np.int32)
        w = np.zeros((T, k), np.float64)
        rc = self.lib.oracle_route_topk(_ptr(logits), T, E, int(k), int(score_fn),
                                        int(bool(renorm)), _ptr(ids), _ptr(w))
        if rc != 0:
            raise ValueError(f"oracle_route_topk failed with {rc}")
        return ids, w

    def router_logits(self, x_bf16: np.ndarray, w_bf16: np.ndarray, nthreads: int = 0) -> np.ndarray:
        """float64[T,E] = x . w^T for bfloat16 bit arrays x[T,H] and w[E,H]."""
        x = _c(x_bf16, np.uint16)
        w = _c(w_bf16, np.uint16)
        T, H = x.shape
        E = w.shape[0]
        assert w.shape[1] == H
        out = np.zeros((T, E), np.float64)
        rc = self.lib.oracle_router_logits(_ptr(x), _ptr(w), T, H, E, int(nthreads), _ptr(out))
        if rc != 0:
            raise ValueError(f"oracle_router_logits failed with {rc}")
        return out

    def group_tokens(self, topk_ids: np.ndarray, E: int) -> dict:
        ids = _c(topk_ids, np.int32)
        T, k = ids.shape
        P = T * k
        out = dict(counts=np.zeros(E, np.int32), offsets=np.zeros(E + 1, np.int32),
                   sorted_pair=np.zeros(max(P, 1), np.int32), pair_pos=np.zeros(max(P, 1), np.int32),
                   active=np.zeros(E, np.int32), n_active=np.zeros(1, np.int32))
        rc = self.lib.oracle_group_tokens(_ptr(ids), T, k, int(E), _ptr(out["counts"]),
                                          _ptr(out["offsets"]), _ptr(out["sorted_pair"]),
                                          _ptr(out["pair_pos"]), _ptr(out["active"]),
                                          _ptr(out["n_active"]))
        if rc != 0:
            raise ValueError(f"oracle_group_tokens failed with {rc}")
        out["sorted_pair"] = out["sorted_pair"][:P]
        out["pair_pos"] = out["pair_pos"][:P]
        out["active"] = out["active"][: int(out["n_active"][0])]
        return out

    def mxfp4_ffn(self, x_bf16: np.ndarray, w13_q, w13_s, w2_q, w2_s, topk_ids, topk_w,
                  clamp_limit: float = 0.0, nthreads: int = 0, want_pairs: bool = False,
                  act_fmt: int = ACT_NONE, want_h: bool = False) -> dict:
        """Expert FFN plus combine. Returns dict(out_ref f64[T,H], out_bf16 u16[T,H], y_pairs?, h_pairs?).
        act_fmt ACT_MXFP8 / ACT_MXFP4 quantises x (per 32 along H) and h (per 32 along I) first;
        want_h returns each pair's h before that quantisation (f64[T*k, I])."""
        x = _c(x_bf16, np.uint16)
        T, H = x.shape
        w13_q = _c(w13_q, np.uint8)
        w13_s = _c(w13_s, np.uint8)
        w2_q = _c(w2_q, np.uint8)
        w2_s = _c(w2_s, np.uint8)
        E, twoI, _ = w13_q.shape
        I = twoI // 2
        ids = _c(topk_ids, np.int32)
        w = _c(topk_w, np.float64)
        k = ids.shape[1]
        assert ids.shape == (T, k) and w.shape == (T, k)
        assert w13_q.shape == (E, 2 * I, H // 2) and w13_s.shape == (E, 2 * I, H // 32)
        assert w2_q.shape == (E, H, I // 2) and w2_s.shape == (E, H, I // 32)
        out_ref = np.zeros((T, H), np.float64)
        out_bf16 = np.zeros((T, H), np.uint16)
        y = np.zeros((T * k, H), np.float64) if want_pairs else None
        hp = np.zeros((T * k, I), np.float64) if want_h else None
        if act_fmt == ACT_NONE and not want_h:
            rc = self.lib.oracle_mxfp4_ffn(_ptr(x), T, H, I, E, k, _ptr(w13_q), _ptr(w13_s),
                                           _ptr(w2_q), _ptr(w2_s), _ptr(ids), _ptr(w),
                                           float(clamp_limit), int(nthreads),
                                           _ptr(y) if y is not None else None, _ptr(out_ref),
                                           _ptr(out_bf16))
        else:
            rc = self.lib.oracle_mxfp4_ffn_act(_ptr(x), T, H, I, E, k, _ptr(w13_q), _ptr(w13_s),
                                               _ptr(w2_q), _ptr(w2_s), _ptr(ids), _ptr(w),
                                               float(clamp_limit), int(act_fmt), int(nthreads),
                                               _ptr(y) if y is not None else None,
                                               _ptr(hp) if hp is not None else None, _ptr(out_ref),
                                               _ptr(out_bf16))
        if rc != 0:
            raise ValueError(f"oracle_mxfp4_ffn failed with {rc}")
        res = dict(out_ref=out_ref, out_bf16=out_bf16)
        if y is not None:
            res["y_pairs"] = y
        if hp is not None:
            res["h_pairs"] = hp
        return res

    def moe_layer(self, logits, x_bf16, w13_q, w13_s, w2_q, w2_s, k, score_fn=SCORE_SOFTMAX,
                  renorm=True, clamp_limit=0.0, nthreads=0, act_fmt=ACT_NONE) -> dict:
        """The whole path: route, group, expert FFN and combine."""
        E = np.asarray(logits).shape[1]
        ids, w = self.route_topk(logits, k, score_fn, renorm)
        grp = self.group_tokens(ids, E)
        ffn = self.mxfp4_ffn(x_bf16, w13_q, w13_s, w2_q, w2_s, ids, w, clamp_limit, nthreads,
                             act_fmt=act_fmt)
        return dict(topk_ids=ids, topk_w=w, **grp, **ffn)

    def num_threads(self, nthreads: int = 0) -> int:
        return int(self.lib.oracle_num_threads(int(nthreads)))


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def default() -> OracleLib:
    """The oracle built from ``moe_oracle.c`` (rebuilt when the source is newer)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _lib = OracleLib(_LIB_PATH)
    return _lib


def e2m1_value(code):
    return default().e2m1_value(code)


def e8m0_value(byte):
    return default().e8m0_value(byte)


def bf16_to_float(bits):
    return default().bf16_to_float(bits)


def float_to_bf16(v):
    return default().float_to_bf16(v)


def mxfp4_element(q, s, K, n, kk):
    return default().mxfp4_element(q, s, K, n, kk)


def e4m3_value(code):
    return default().e4m3_value(code)


def e4m3_encode(v):
    return default().e4m3_encode(v)


def e2m1_encode(v):
    return default().e2m1_encode(v)


def mx_element(fmt, code):
    return default().mx_element(fmt, code)


def mx_quantize_block(v, fmt):
    return default().mx_quantize_block(v, fmt)


def mx_dequantize(v, fmt):
    return default().mx_dequantize(v, fmt)


def route_topk(logits, k, score_fn=SCORE_SOFTMAX, renorm=True):
    return default().route_topk(logits, k, score_fn, renorm)


def group_tokens(topk_ids, E):
    return default().group_tokens(topk_ids, E)


def router_logits(x_bf16, w_bf16, nthreads=0):
    return default().router_logits(x_bf16, w_bf16, nthreads)


def mxfp4_ffn(x_bf16, w13_q, w13_s, w2_q, w2_s, topk_ids, topk_w, clamp_limit=0.0, nthreads=0,
              want_pairs=False, act_fmt=ACT_NONE, want_h=False):
    return default().mxfp4_ffn(x_bf16, w13_q, w13_s, w2_q, w2_s, topk_ids, topk_w, clamp_limit,
                               nthreads, want_pairs, act_fmt, want_h)


def moe_layer(logits, x_bf16, w13_q, w13_s, w2_q, w2_s, k, score_fn=SCORE_SOFTMAX, renorm=True,
              clamp_limit=0.0, nthreads=0, act_fmt=ACT_NONE):
    return default().moe_layer(logits, x_bf16, w13_q, w13_s, w2_q, w2_s, k, score_fn, renorm,
                               clamp_limit, nthreads, act_fmt)


def num_threads(nthreads: int = 0) -> int:
    return default().num_threads(nthreads)
