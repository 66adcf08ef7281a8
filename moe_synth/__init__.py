"""Seeded synthetic inputs for the routed MXFP4 MoE feed-forward.

This module holds only input generation: shapes, value distributions and seeds. It contains none of
the method's arithmetic (no decoding, routing, grouping or GEMM) and is shared by the tests, the
benchmark and the smoke check, which feed the same arrays to the CPU oracle and to the HIP library.

Workloads (the pages measure decode at concurrency 1, 10, 256 and 1024 on Blackwell — "Chunk 8.0";
c8 decode at matched M=8 — vllm.cpp PR #52; MTP1 decode with M=2 — "MTP1 Post-Portfolio Eager-Cycle
Profile"; no dataset or weights are used, every value is drawn here):

  name           T     H     I     E    k  routing            logits
  tiny           4   256   128     8    2  softmax, renorm    N(0,1)
  decode_c1      1  2048   768   128    8  softmax, renorm    N(0,1)
  decode_m2      2  4096  2048   256    8  softmax, renorm    U[-1,1)
  decode_m8      8  4096  2048   256    8  softmax, renorm    U[-1,1)
  medium_zipf  256  4096  2048   256    8  softmax, renorm    N(0,1) + Zipf(1.1) popularity bias
  high_c4     1024  7168  2048   256    8  sigmoid, renorm    N(0,1); gate/up clamped to [-7, 7]
  m1024       1024  7168  2048     8    8  softmax, renorm    N(0,1) (every expert sees every token)

Draw order from numpy PCG64(seed): logits, x, w13 codes, w13 scales, w2 codes, w2 scales, then the
Zipf expert-rank permutation. x is N(0,1) rounded to bfloat16 (nearest-even). Codes are uniform bytes
(both nibbles uniform over the 16 E2M1 codes); scales are integers uniform in [120, 124].
"""
from __future__ import annotations

import dataclasses

import numpy as np

SEED_BASE = 20261203
SCORE_SOFTMAX = 0
SCORE_SIGMOID = 1


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    T: int
    H: int
    I: int
    E: int
    k: int
    score_fn: int = SCORE_SOFTMAX
    renorm: bool = True
    clamp: float = 0.0
    logits: str = "normal"  # normal | uniform | zipf
    index: int = 0

    @property
    def P(self) -> int:
        return self.T * self.k

    def with_tokens(self, T: int) -> "Config":
        return dataclasses.replace(self, T=T)


CONFIGS = {
    c.name: c
    for c in [
        Config("tiny", 4, 256, 128, 8, 2, index=0),
        Config("decode_c1", 1, 2048, 768, 128, 8, index=1),
        Config("decode_m2", 2, 4096, 2048, 256, 8, logits="uniform", index=2),
        Config("decode_m8", 8, 4096, 2048, 256, 8, logits="uniform", index=2),
        Config("medium_zipf", 256, 4096, 2048, 256, 8, logits="zipf", index=3),
        Config("high_c4", 1024, 7168, 2048, 256, 8, score_fn=SCORE_SIGMOID, clamp=7.0,
               logits="normal", index=4),
        Config("m1024", 1024, 7168, 2048, 8, 8, index=5),
    ]
}

ZIPF_S = 1.1
ZIPF_BETA = 0.25


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even) and return the 16-bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def zipf_bias(E: int, rank_perm: np.ndarray, s: float = ZIPF_S, beta: float = ZIPF_BETA) -> np.ndarray:
    """Per-expert logit bias beta*ln(E*p_rank) with p_r proportional to r^-s over ranks 1..E."""
    r = np.arange(1, E + 1, dtype=np.float64)
    p = r ** (-s)
    p /= p.sum()
    return (beta * np.log(E * p[rank_perm])).astype(np.float32)


def make_inputs(cfg: Config, seed: int | None = None, weights: bool = True,
                scale_lo: int = 120, scale_hi: int = 124) -> dict:
    """Draw one workload. Returns numpy arrays; weights are omitted when ``weights`` is False."""
    rng = np.random.Generator(np.random.PCG64(SEED_BASE + cfg.index if seed is None else seed))
    T, H, I, E = cfg.T, cfg.H, cfg.I, cfg.E
    if cfg.logits == "uniform":
        logits = rng.uniform(-1.0, 1.0, size=(T, E)).astype(np.float32)
    else:
        logits = rng.standard_normal(size=(T, E), dtype=np.float32)
    x = f32_to_bf16_bits(rng.standard_normal(size=(T, H), dtype=np.float32))
    out = dict(logits=logits, x=x)
    if weights:
        out["w13_q"] = rng.integers(0, 256, size=(E, 2 * I, H // 2), dtype=np.uint8)
        out["w13_s"] = rng.integers(scale_lo, scale_hi + 1, size=(E, 2 * I, H // 32), dtype=np.uint8)
        out["w2_q"] = rng.integers(0, 256, size=(E, H, I // 2), dtype=np.uint8)
        out["w2_s"] = rng.integers(scale_lo, scale_hi + 1, size=(E, H, I // 32), dtype=np.uint8)
    if cfg.logits == "zipf":
        perm = rng.permutation(E)
        out["logits"] = (logits + zipf_bias(E, perm)[None, :]).astype(np.float32)
        out["zipf_rank"] = perm
    return out


def make_weights(E: int, H: int, I: int, seed: int, scale_lo: int = 120, scale_hi: int = 124) -> dict:
    """Weights only, from their own seed (used for small random-shape cases)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return dict(
        w13_q=rng.integers(0, 256, size=(E, 2 * I, H // 2), dtype=np.uint8),
        w13_s=rng.integers(scale_lo, scale_hi + 1, size=(E, 2 * I, H // 32), dtype=np.uint8),
        w2_q=rng.integers(0, 256, size=(E, H, I // 2), dtype=np.uint8),
        w2_s=rng.integers(scale_lo, scale_hi + 1, size=(E, H, I // 32), dtype=np.uint8),
    )


def make_router_weights(E: int, H: int, seed: int) -> np.ndarray:
    """Router weights W_router[E, H] as bfloat16 bits, N(0, 1/H) from their own seed, so that with
    N(0, 1) activations the logits are about N(0, 1), like the logits the configs draw directly."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return f32_to_bf16_bits((rng.standard_normal(size=(E, H), dtype=np.float32) / np.float32(np.sqrt(H))))


def small_case(T: int, H: int, I: int, E: int, k: int, seed: int, logits: str = "normal",
               score_fn: int = SCORE_SOFTMAX, clamp: float = 0.0, scale_lo: int = 120,
               scale_hi: int = 124) -> tuple[Config, dict]:
    """A random small workload with explicit shape (ragged shapes, edge cases); scale bytes uniform
    in [scale_lo, scale_hi]."""
    cfg = Config(f"case_T{T}_H{H}_I{I}_E{E}_k{k}_s{seed}", T, H, I, E, k, score_fn=score_fn,
                 clamp=clamp, logits=logits)
    return cfg, make_inputs(cfg, seed=seed, scale_lo=scale_lo, scale_hi=scale_hi)


def lower_one_block_per_row(s: np.ndarray, below: int, seed: int) -> np.ndarray:
    """Scale bytes [E, N, K/32] (K/32 >= 2) with one block of every row (a seeded choice) set `below`
    steps under the largest byte of the row's other blocks (at least 2), the rest unchanged."""
    rng = np.random.Generator(np.random.PCG64(seed))
    s = s.copy()
    E, N, nb = s.shape
    assert nb >= 2
    pick = rng.integers(0, nb, size=(E, N))
    others = s.astype(np.int64)
    np.put_along_axis(others, pick[..., None], -1, axis=2)
    low = np.maximum(others.max(axis=2) - below, 2).astype(np.uint8)
    np.put_along_axis(s, pick[..., None], low[..., None], axis=2)
    return s


def extreme_scale_case(T: int, H: int, I: int, E: int, k: int, seed: int, lam=(0, 20, -20, 100),
                       score_fn: int = SCORE_SOFTMAX) -> tuple[Config, dict]:
    """Weights whose E8M0 scale bytes reach both ends of the range the device decodes exactly (2 and
    252), with activations that offset them so that no product or sum leaves the binary32 range.

      - every fourth H-block of x holds values +-(1 + U[0,1)) * 2^-125 (normal bfloat16); the gate rows'
        scale bytes in those blocks are 252 (products of ordinary size), elsewhere x ~ N(0,1) and the
        gate scale bytes are 127 + U{-2..2}, with byte 2 in every fifth block (products ~2^-125);
      - the up rows of I-block j carry an offset lam[j % len(lam)]: scale byte 127 + d - lam (kept in
        [2, 252]), d = 125 on the 2^-125 x blocks and 0 elsewhere, so u (and h) of those rows is about
        2^-lam;
      - the down rows' scale bytes in I-block j are 127 + lam[j % len(lam)] + U{-2..2}, which brings each
        block's products back to ordinary size, except: byte 252 in every third I-block whose lam is the
        largest (products ~2^(125 - lam): those blocks dominate the output) and byte 2 in every seventh
        block.
    Codes are uniform bytes, logits N(0,1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    cfg = Config(f"extreme_T{T}_H{H}_I{I}_E{E}_k{k}_s{seed}", T, H, I, E, k, score_fn=score_fn)
    nbh, nbi = H // 32, I // 32
    logits = rng.standard_normal(size=(T, E), dtype=np.float32)
    d = np.where(np.arange(nbh) % 4 == 1, 125, 0)  # x exponent offset per H-block
    mag = (1.0 + rng.random(size=(T, H))) * np.where(rng.random(size=(T, H)) < 0.5, -1.0, 1.0)
    x = np.where(np.repeat(d, 32)[None, :] == 125, mag * 2.0 ** -125,
                 rng.standard_normal(size=(T, H))).astype(np.float32)
    lam_i = np.array([lam[j % len(lam)] for j in range(nbi)])  # per I-block of h
    jit = lambda shape: rng.integers(-2, 3, size=shape)  # noqa: E731
    gate_s = np.where(d[None, None, :] == 125, 252, 127 + jit((E, I, nbh)))
    gate_s = np.where((np.arange(nbh) % 5 == 3)[None, None, :] & (d[None, None, :] == 0), 2, gate_s)
    up_lam = np.repeat(lam_i, 32)[:I]  # per up row
    up_s = np.broadcast_to(np.clip(127 + d[None, None, :] - up_lam[None, :, None], 2, 252), (E, I, nbh))
    w2_s = 127 + lam_i[None, None, :] + jit((E, H, nbi))
    w2_s = np.where(((np.arange(nbi) % 3 == 0) & (lam_i == max(lam)))[None, None, :], 252, w2_s)
    w2_s = np.where((np.arange(nbi) % 7 == 5)[None, None, :], 2, w2_s)
    w13_s = np.concatenate([gate_s, up_s], axis=1)
    assert w13_s.min() >= 2 and w13_s.max() <= 252 and w2_s.min() >= 2 and w2_s.max() <= 252
    out = dict(logits=logits, x=f32_to_bf16_bits(x),
               w13_q=rng.integers(0, 256, size=(E, 2 * I, H // 2), dtype=np.uint8),
               w13_s=w13_s.astype(np.uint8),
               w2_q=rng.integers(0, 256, size=(E, H, I // 2), dtype=np.uint8),
               w2_s=w2_s.astype(np.uint8))
    return cfg, out


def active_weight_bytes(counts: np.ndarray, H: int, I: int) -> int:
    """Weight bytes the layer must stream: every expert with at least one routed pair reads its
    3*H*I codes (half a byte each) and 3*H*I/32 scale bytes."""
    n_active = int(np.count_nonzero(np.asarray(counts)))
    per_expert = 3 * H * I // 2 + 3 * H * I // 32
    return n_active * per_expert
