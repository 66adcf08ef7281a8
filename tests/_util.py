"""Test helpers that are independent of both the oracle and the HIP library.

The MXFP4 dequantiser here is a second, table-driven implementation written from the OCP
Microscaling Formats (MX) v1.0 MXFP4 definition (the E2M1 value table and the E8M0 scale 2^(s-127)),
used to pin the oracle's own formula-driven decoder.
"""
import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# Magnitudes of the eight non-negative E2M1 codes, as tabulated in the OCP MX v1.0 specification.
E2M1_TABLE = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], np.float64)


def dequant(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """[..., N, K/2] packed codes + [..., N, K/32] scales -> float64 [..., N, K]."""
    q = np.asarray(q, np.uint8)
    lo = q & 0xF
    hi = q >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(*q.shape[:-1], q.shape[-1] * 2)
    mag = E2M1_TABLE[codes & 7]
    val = np.where(codes & 8, -mag, mag)
    scale = np.exp2(np.asarray(s, np.float64) - 127.0)
    scale = np.where(np.asarray(s) == 255, np.nan, scale)
    return val * np.repeat(scale, 32, axis=-1)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def load_golden(name: str) -> dict:
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def golden_value(v):
    if isinstance(v, str):
        if v == "ln3":
            return math.log(3.0)
        num, den = v.split("/")
        return float(num) / float(den)
    return float(v)


def build_golden_inputs(g: dict) -> dict:
    sh = g["shape"]
    T, H, I, E, k = sh["T"], sh["H"], sh["I"], sh["E"], sh["k"]
    logits = np.array([[golden_value(v) for v in row] for row in g["logits"]], np.float32)
    x = np.zeros((T, H), np.float32)
    for t, h, v in g["x_nonzero"]:
        x[t, h] = v
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)  # exact: the values are bfloat16-representable
    w13_q = np.full((E, 2 * I, H // 2), g["default_code_byte"], np.uint8)
    w13_s = np.full((E, 2 * I, H // 32), g["default_scale_byte"], np.uint8)
    w2_q = np.full((E, H, I // 2), g["default_code_byte"], np.uint8)
    w2_s = np.full((E, H, I // 32), g["default_scale_byte"], np.uint8)
    for e, r, b, v in g.get("w13_code_bytes", []):
        w13_q[e, r, b] = v
    for e, r, b, v in g.get("w13_scale_bytes", []):
        w13_s[e, r, b] = v
    for e, r, b, v in g.get("w2_code_bytes", []):
        w2_q[e, r, b] = v
    for e, r, b, v in g.get("w2_scale_bytes", []):
        w2_s[e, r, b] = v
    return dict(logits=logits, x=xb, w13_q=w13_q, w13_s=w13_s, w2_q=w2_q, w2_s=w2_s,
                T=T, H=H, I=I, E=E, k=k, score_fn=0 if g["score_fn"] == "softmax" else 1,
                renorm=g["renorm"], clamp=g["clamp"])


def numpy_bruteforce_ffn(x_bits, w13_q, w13_s, w2_q, w2_s, ids, w, clamp=0.0):
    """Per-token loop over the selected experts with whole-matrix dequantisation and numpy matmuls."""
    x = bf16_to_f64(x_bits)
    T, H = x.shape
    E, twoI, _ = w13_q.shape
    I = twoI // 2
    out = np.zeros((T, H), np.float64)
    for t in range(T):
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            W13 = dequant(w13_q[e], w13_s[e])
            W2 = dequant(w2_q[e], w2_s[e])
            g = W13[:I] @ x[t]
            u = W13[I:] @ x[t]
            if clamp > 0:
                g = np.clip(g, -clamp, clamp)
                u = np.clip(u, -clamp, clamp)
            h = g / (1.0 + np.exp(-g)) * u
            out[t] += w[t, j] * (W2 @ h)
    return out


def rne_bf16(ref: np.ndarray) -> np.ndarray:
    """ref rounded to bfloat16 (nearest-even) as float64, via torch's CPU conversion."""
    import torch

    return torch.from_numpy(np.asarray(ref, np.float64)).to(torch.bfloat16).to(torch.float64).numpy()


def parity_metrics(out_bf16_bits, ref):
    """Error of a bfloat16 output against the unrounded fp64 oracle output `ref`:
      max_raw    = max |out - ref| / rms(ref)
      max_excess = max (|out - ref| - |bf16(ref) - ref|) / rms(ref): the error beyond what rounding
                   the exact value to bfloat16 already costs at that element
      l1         = sum |out - ref| / sum |ref|
    """
    out = bf16_to_f64(out_bf16_bits)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return dict(max_raw=0.0, max_excess=0.0, l1=0.0)
    err = np.abs(out - ref)
    own = np.abs(rne_bf16(ref) - ref)
    rms = math.sqrt(float(np.mean(ref * ref)))
    den = float(np.abs(ref).sum())
    return dict(max_raw=float(err.max()) / rms if rms > 0 else float(err.max()),
                max_excess=float((err - own).max()) / rms if rms > 0 else float((err - own).max()),
                l1=float(err.sum()) / den if den > 0 else float(err.sum()))


# ---- MX activation quantisers of the tests (independent of the oracle's) -------------------------

ACT_MXFP8 = 1
ACT_MXFP4 = 2


def e4m3_torch(v):
    """Nearest E4M3 values (ties to even) of v, saturating at 448, via torch's conversion. torch
    converts a float64 through binary32, so v must be binary32 values for a single rounding."""
    import torch

    v = np.clip(np.asarray(v, np.float64), -448.0, 448.0)
    return torch.from_numpy(v).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def e2m1_bruteforce(v):
    """Nearest E2M1 values by a search over the eight magnitudes (a tie, always between neighbouring
    codes, goes to the even code), saturating at 6."""
    v = np.asarray(v, np.float64)
    a = np.minimum(np.abs(v), 6.0)
    d = np.abs(a[..., None] - E2M1_TABLE)
    cand = d == d.min(axis=-1, keepdims=True)
    rank = np.where(cand, np.arange(8) % 2, 2)  # an even candidate first, else the only one
    return np.copysign(E2M1_TABLE[rank.argmin(axis=-1)], v)


def mx_fake_quant(v, fmt):
    """Blocks of 32 along the last axis: scale 2^(floor(log2 amax) - emax), clamped to [-127, 127],
    then each element rounded by the element quantiser above."""
    v = np.asarray(v, np.float64)
    b = v.reshape(-1, 32)
    amax = np.abs(b).max(axis=1)
    emax = 8 if fmt == ACT_MXFP8 else 2
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))
    shared = np.clip(e - 1 - emax, -127, 127).astype(np.float64)
    X = np.exp2(shared)[:, None]
    q = e4m3_torch(b / X) if fmt == ACT_MXFP8 else e2m1_bruteforce(b / X)
    q = np.where(amax[:, None] > 0, q * X, 0.0)
    return q.reshape(v.shape)
