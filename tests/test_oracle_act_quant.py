"""Pins for the oracle's activation-quantised mode (MX blocks of 32 values, MXFP8 and MXFP4).

* E4M3 decoding of all 256 codes and encoding of random values, every tie and the saturation range
  against torch's float8_e4m3fn conversion (a library routine);
* E2M1 encoding against a brute-force nearest search over the specification's value table;
* hand-worked blocks (tests/golden/mx_blocks.json) for the shared scale, rounding, saturation, the
  scale clamp and the zero block;
* round trips of blocks that are exactly representable, idempotence, scale equivariance and the
  element error bound;
* the whole FFN: E=1, k=1 is the dense SwiGLU MLP on quantised activations (the test's own quantiser:
  torch's E4M3 cast resp. the brute-force E2M1 search), a numpy per-token loop on random shapes, the
  reduction to the unquantised FFN on representable inputs, and a pin of the binary32 rounding of h
  before its quantisation.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import moe_synth
from _util import GOLDEN, E2M1_TABLE, bf16_to_f64, dequant, e2m1_bruteforce, e4m3_torch, mx_fake_quant

from _util import ACT_MXFP4, ACT_MXFP8

FMT = {"mxfp8": ACT_MXFP8, "mxfp4": ACT_MXFP4}


def test_e2m1_bruteforce_itself_on_ties():
    # the test's quantiser on the midpoints: 0.25->0, 0.75->1, 1.25->1, 1.75->2, 2.5->2, 3.5->4, 5->4
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, -0.75])
    np.testing.assert_array_equal(e2m1_bruteforce(mids), [0, 1, 1, 2, 2, 4, 4, 6, -1])


# ---- element formats ------------------------------------------------------------------------------

def test_e4m3_decode_all_codes_match_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([orc.e4m3_value(c) for c in codes])
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))
    # landmarks of the format: largest normal, smallest normal, largest and smallest subnormal
    assert orc.e4m3_value(0x7E) == 448.0 and orc.e4m3_value(0x08) == 2.0 ** -6
    assert orc.e4m3_value(0x07) == 7 * 2.0 ** -9 and orc.e4m3_value(0x01) == 2.0 ** -9
    assert math.isnan(orc.e4m3_value(0x7F)) and math.isnan(orc.e4m3_value(0xFF))


def _e4m3_code_torch(v):
    v = np.clip(np.asarray(v, np.float64), -448.0, 448.0)
    return torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_matches_torch(orc):
    rng = np.random.default_rng(3)
    v = (rng.standard_normal(6000) * np.exp2(rng.uniform(-14, 10, 6000))).astype(np.float32).astype(np.float64)
    finite = np.array([orc.e4m3_value(c) for c in range(127)])
    mids = (finite[1:] + finite[:-1]) / 2  # every tie between neighbouring codes
    v = np.concatenate([v, mids, -mids, [0.0, -0.0, 448.0, 449.0, 464.0, 479.9, 480.0, 1e9, -1e9]])
    got = np.array([orc.e4m3_encode(x) for x in v], np.uint8)
    np.testing.assert_array_equal(got, _e4m3_code_torch(v))


def test_e2m1_encode_matches_bruteforce(orc):
    rng = np.random.default_rng(4)
    v = np.concatenate([np.arange(-128, 129) / 16.0, rng.uniform(-8, 8, 3000), [1e9, -1e9, -0.0]])
    got = np.array([orc.e2m1_value(orc.e2m1_encode(x)) for x in v])
    ref = e2m1_bruteforce(v)
    np.testing.assert_array_equal(got, ref)
    # the sign of a negative value that rounds to zero is kept (code 8)
    assert orc.e2m1_encode(-0.1) == 8 and orc.e2m1_encode(0.1) == 0


# ---- blocks ---------------------------------------------------------------------------------------

def _golden_value(s):
    s = s.strip()
    if "2^" in s:
        coef, _, ex = s.partition("2^")
        c = float(coef.rstrip("*")) if coef else 1.0
        return c * 2.0 ** int(ex)
    return float(s)


with open(os.path.join(GOLDEN, "mx_blocks.json")) as _f:
    _BLOCKS = json.load(_f)["blocks"]


@pytest.mark.parametrize("blk", _BLOCKS, ids=lambda b: b["name"])
def test_golden_block(orc, blk):
    fmt = FMT[blk["fmt"]]
    v = np.zeros(32)
    for i, s in blk["values"]:
        v[i] = _golden_value(s)
    if "-0.0" in [s for _, s in blk["values"]]:
        v[[i for i, s in blk["values"] if s == "-0.0"]] = -0.0
    want = np.zeros(32, np.uint8)
    for i, c in blk["codes"]:
        want[i] = int(c, 16)
    scale, codes = orc.mx_quantize_block(v, fmt)
    assert scale == blk["scale_byte"]
    np.testing.assert_array_equal(codes, want)


@pytest.mark.parametrize("fmt", [ACT_MXFP8, ACT_MXFP4])
def test_representable_blocks_round_trip(orc, fmt):
    """A block whose elements are codes of the format times 2^s, with at least one element in the
    format's top binade, is quantised back to exactly those codes and the scale byte s + 127."""
    rng = np.random.default_rng(5 + fmt)
    for trial in range(200):
        s = int(rng.integers(-120, 120))
        if fmt == ACT_MXFP8:
            codes = rng.integers(0, 256, 32).astype(np.uint8)
            codes[(codes & 0x7F) == 0x7F] = 0x10  # no NaN codes
            top = int(rng.integers(0, 32))
            codes[top] = (codes[top] & 0x80) | (0x78 | int(rng.integers(0, 7)))  # exponent field 15
        else:
            codes = rng.integers(0, 16, 32).astype(np.uint8)
            top = int(rng.integers(0, 32))
            codes[top] = (codes[top] & 8) | int(rng.integers(6, 8))  # magnitude 4 or 6
        v = np.array([orc.mx_element(fmt, c) for c in codes]) * 2.0 ** s
        scale, got = orc.mx_quantize_block(v, fmt)
        assert scale == s + 127
        np.testing.assert_array_equal(got, codes)


@pytest.mark.parametrize("fmt", [ACT_MXFP8, ACT_MXFP4])
def test_block_idempotent_equivariant_and_bounded(orc, fmt):
    rng = np.random.default_rng(11 + fmt)
    v = rng.standard_normal((40, 32)) * np.exp2(rng.uniform(-20, 20, (40, 1)))
    v[3, :] = 0.0
    v[4, 5:] = 0.0
    q = orc.mx_dequantize(v, fmt)
    np.testing.assert_array_equal(orc.mx_dequantize(q, fmt), q)
    for j in (-3, 1, 7):
        np.testing.assert_array_equal(orc.mx_dequantize(v * 2.0 ** j, fmt), q * 2.0 ** j)
    # element error: at most half a spacing of the element grid at the block's scale, except where the
    # scaled value exceeds the largest normal (saturation)
    mbits, emin, vmax = (3, -6, 448.0) if fmt == ACT_MXFP8 else (1, 0, 6.0)
    emax = 8 if fmt == ACT_MXFP8 else 2
    for b in range(v.shape[0]):
        amax = np.abs(v[b]).max()
        if amax == 0:
            assert np.all(q[b] == 0)
            continue
        X = 2.0 ** (math.floor(math.log2(amax)) - emax)
        a = np.abs(v[b]) / X
        ex = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), emin)
        half = 2.0 ** (ex - mbits) / 2 * X
        sat = a > vmax
        assert np.all(np.abs(q[b] - v[b])[~sat] <= half[~sat])
        assert np.all(np.abs(q[b][sat]) == vmax * X)


def test_matches_test_quantiser_on_random_blocks(orc):
    rng = np.random.default_rng(21)
    for fmt in (ACT_MXFP8, ACT_MXFP4):
        v = (rng.standard_normal((64, 32)) * np.exp2(rng.uniform(-30, 30, (64, 1)))).astype(np.float32)
        v = v.astype(np.float64)
        np.testing.assert_array_equal(orc.mx_dequantize(v, fmt), mx_fake_quant(v, fmt))


# ---- the FFN in the activation-quantised mode -----------------------------------------------------

def _h32(h):
    return h.astype(np.float32).astype(np.float64)


@pytest.mark.parametrize("fmt", [ACT_MXFP8, ACT_MXFP4])
@pytest.mark.parametrize("H,I,clamp", [(64, 32, 0.0), (96, 160, 0.0), (256, 128, 3.0)])
def test_single_expert_is_dense_mlp_on_quantised_activations(orc, fmt, H, I, clamp):
    T = 5
    rng = np.random.default_rng(H + I + fmt)
    x = moe_synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    w = moe_synth.make_weights(1, H, I, seed=H * 7 + I)
    ids = np.zeros((T, 1), np.int32)
    wt = np.ones((T, 1))
    res = orc.mxfp4_ffn(x, w["w13_q"], w["w13_s"], w["w2_q"], w["w2_s"], ids, wt, clamp, act_fmt=fmt)
    X = torch.from_numpy(mx_fake_quant(bf16_to_f64(x), fmt))
    W13 = torch.from_numpy(dequant(w["w13_q"][0], w["w13_s"][0]))
    W2 = torch.from_numpy(dequant(w["w2_q"][0], w["w2_s"][0]))
    gate = X @ W13[:I].T
    up = X @ W13[I:].T
    if clamp > 0:
        gate = gate.clamp(-clamp, clamp)
        up = up.clamp(-clamp, clamp)
    h = torch.from_numpy(mx_fake_quant(_h32((torch.nn.functional.silu(gate) * up).numpy()), fmt))
    ref = h @ W2.T
    np.testing.assert_allclose(res["out_ref"], ref.numpy(), rtol=1e-12, atol=1e-12 * float(ref.abs().max()))
    # and it differs from the unquantised FFN by the quantisation error, not by nothing
    plain = orc.mxfp4_ffn(x, w["w13_q"], w["w13_s"], w["w2_q"], w["w2_s"], ids, wt, clamp)["out_ref"]
    rel = np.abs(res["out_ref"] - plain).max() / np.abs(plain).max()
    assert 1e-4 < rel < (0.2 if fmt == ACT_MXFP8 else 1.0)


@pytest.mark.parametrize("fmt", [ACT_MXFP8, ACT_MXFP4])
@pytest.mark.parametrize("T,H,I,E,k,score_fn,clamp,seed", [
    (4, 256, 128, 8, 2, 0, 0.0, 0),
    (6, 128, 64, 8, 3, 1, 7.0, 2),
    (7, 96, 32, 16, 4, 0, 2.5, 4),
])
def test_act_mode_matches_numpy_per_token_loop(orc, fmt, T, H, I, E, k, score_fn, clamp, seed):
    cfg, inp = moe_synth.small_case(T, H, I, E, k, seed, score_fn=score_fn, clamp=clamp)
    ids, w = orc.route_topk(inp["logits"], k, score_fn)
    res = orc.mxfp4_ffn(inp["x"], inp["w13_q"], inp["w13_s"], inp["w2_q"], inp["w2_s"], ids, w, clamp,
                        act_fmt=fmt, want_pairs=True)
    xq = mx_fake_quant(bf16_to_f64(inp["x"]), fmt)
    out = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            W13 = dequant(inp["w13_q"][e], inp["w13_s"][e])
            W2 = dequant(inp["w2_q"][e], inp["w2_s"][e])
            g, u = W13[:I] @ xq[t], W13[I:] @ xq[t]
            if clamp > 0:
                g, u = np.clip(g, -clamp, clamp), np.clip(u, -clamp, clamp)
            y = W2 @ mx_fake_quant(_h32(g / (1.0 + np.exp(-g)) * u), fmt)
            np.testing.assert_allclose(res["y_pairs"][t * k + j], y, rtol=1e-11, atol=1e-11 * np.abs(y).max())
            out[t] += w[t, j] * y
    np.testing.assert_allclose(res["out_ref"], out, rtol=1e-11, atol=1e-11 * float(np.abs(out).max()))


def test_act_none_is_the_plain_ffn(orc):
    cfg, inp = moe_synth.small_case(5, 128, 64, 6, 3, 9)
    ids, w = orc.route_topk(inp["logits"], 3)
    a = orc.mxfp4_ffn(inp["x"], inp["w13_q"], inp["w13_s"], inp["w2_q"], inp["w2_s"], ids, w)
    b = orc.mxfp4_ffn(inp["x"], inp["w13_q"], inp["w13_s"], inp["w2_q"], inp["w2_s"], ids, w, act_fmt=0)
    np.testing.assert_array_equal(a["out_ref"], b["out_ref"])


def test_h_is_rounded_to_binary32_before_its_quantisation(orc):
    """A constructed case where the decision depends on it: g = 20.0390625/256 and u = -52.25/256 give
    h = silu(g)*u = -0.0083007814486..., whose binary32 rounding is exactly -(272/256)*2^-7, the tie
    between the E4M3 codes 256 and 288 at the block scale 2^-15 (h is alone in its block). From binary32
    the tie goes to the even code, 256, so out = -2^-7; from the fp64 value it would round up to 288."""
    T, H, I, E = 1, 32, 32, 1
    x = np.zeros((T, H), np.float32)
    x[0, :4] = [0.0390625, 20.0, -52.0, -0.25]
    x[0, 31] = 256.0  # the block's largest magnitude: x's block scale is 1, every x is an E4M3 value
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    w13_q = np.zeros((E, 2 * I, H // 2), np.uint8)
    w13_s = np.full((E, 2 * I, H // 32), 127, np.uint8)
    w13_q[0, 0, 0] = 0x22      # gate row 0: weight 1 on x[0] and x[1] ...
    w13_s[0, 0, 0] = 127 - 8   # ... times 2^-8
    w13_q[0, I, 1] = 0x22      # up row 0: weight 1 on x[2] and x[3], times 2^-8
    w13_s[0, I, 0] = 127 - 8
    w2_q = np.zeros((E, H, I // 2), np.uint8)
    w2_q[0, :, 0] = 0x02       # every output: weight 1 on h[0]
    w2_s = np.full((E, H, I // 32), 127, np.uint8)
    g, u = 20.0390625 / 256, -52.25 / 256
    h = g / (1.0 + math.exp(-g)) * u
    assert float(np.float32(h)) == -(272 / 256) * 2.0 ** -7 and h < float(np.float32(h))
    res = orc.mxfp4_ffn(xb, w13_q, w13_s, w2_q, w2_s, np.zeros((T, 1), np.int32), np.ones((T, 1)),
                        act_fmt=ACT_MXFP8)
    np.testing.assert_array_equal(res["out_ref"], np.full((T, H), -2.0 ** -7))
    # the test's own quantiser agrees, and without the binary32 step it would not
    hq = mx_fake_quant(_h32(np.array([h] + [0.0] * 31)), ACT_MXFP8)[0]
    assert hq == -2.0 ** -7
    # from fp64, |h| at the block scale lies above the tie 272, so the nearest E4M3 value is 288
    assert 272.0 < abs(h) * 2.0 ** 15 < 288.0 and abs(h) * 2.0 ** 15 - 272.0 > 1e-6


def test_h_pairs_output(orc):
    """The optional h output is each pair's h before quantisation: binary32 values that quantise to the
    h the down projection uses (checked through y), and, unquantised, the plain FFN's h."""
    cfg, inp = moe_synth.small_case(3, 64, 64, 4, 2, 12)
    ids, w = orc.route_topk(inp["logits"], 2)
    res = orc.mxfp4_ffn(inp["x"], inp["w13_q"], inp["w13_s"], inp["w2_q"], inp["w2_s"], ids, w, act_fmt=ACT_MXFP8,
                        want_pairs=True, want_h=True)
    h = res["h_pairs"]
    np.testing.assert_array_equal(h, _h32(h))
    for p in range(h.shape[0]):
        W2 = dequant(inp["w2_q"][ids.flat[p]], inp["w2_s"][ids.flat[p]])
        np.testing.assert_allclose(res["y_pairs"][p], W2 @ mx_fake_quant(h[p], ACT_MXFP8), rtol=1e-12,
                                   atol=1e-12 * np.abs(res["y_pairs"][p]).max())
    plain = orc.mxfp4_ffn(inp["x"], inp["w13_q"], inp["w13_s"], inp["w2_q"], inp["w2_s"], ids, w, want_h=True)
    xd = bf16_to_f64(inp["x"])
    for p in range(h.shape[0]):
        W13 = dequant(inp["w13_q"][ids.flat[p]], inp["w13_s"][ids.flat[p]])
        g, u = W13[:64] @ xd[p // 2], W13[64:] @ xd[p // 2]
        np.testing.assert_allclose(plain["h_pairs"][p], g / (1 + np.exp(-g)) * u, rtol=1e-12, atol=1e-14)
