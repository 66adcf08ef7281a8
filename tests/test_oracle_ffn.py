"""Pins for the oracle's expert FFN and combine.

* worked examples A and B (tests/golden), checked against closed forms;
* E=1, k=1 reduces to the textbook dense SwiGLU MLP, checked with torch CPU fp64 matmuls on weights
  dequantised by the independent table-driven decoder;
* a numpy brute-force per-token loop on random tiny shapes;
* metamorphic relations that hold exactly in fp64 (scale +1 doubles the output, expert relabelling,
  token permutation).
"""
import math

import numpy as np
import pytest
import torch

import moe_synth
from _util import bf16_to_f64, build_golden_inputs, dequant, load_golden, numpy_bruteforce_ffn


def run_golden(orc, name):
    g = load_golden(name)
    inp = build_golden_inputs(g)
    res = orc.moe_layer(inp["logits"], inp["x"], inp["w13_q"], inp["w13_s"], inp["w2_q"], inp["w2_s"],
                        inp["k"], inp["score_fn"], inp["renorm"], inp["clamp"])
    return g, inp, res


def test_worked_example_a(orc):
    g, inp, res = run_golden(orc, "worked_example_a.json")
    ex = g["expected"]
    np.testing.assert_array_equal(res["topk_ids"], ex["topk_ids"])
    l = float(np.float32(math.log(3.0)))  # the logits are float32
    wa = [math.exp(l) / (1.0 + math.exp(l)), 1.0 / (1.0 + math.exp(l))]
    np.testing.assert_allclose(res["topk_w"][0], wa, rtol=1e-15)
    np.testing.assert_allclose(wa, ex["topk_w_value"], rtol=1e-15)
    assert abs(wa[0] - 0.75) < 1e-8
    for key in ("counts", "offsets", "sorted_pair", "pair_pos", "active"):
        np.testing.assert_array_equal(res[key], ex[key])
    y0 = 0.5 * 2.0 / (1.0 + math.exp(-2.0)) * 1.0
    y1 = 1.0 * (-1.0) / (1.0 + math.exp(1.0)) * 3.0
    want = wa[0] * y1 + wa[1] * y0
    assert abs(want - ex["out_ref_0_1_value"]) < 1e-14
    out = res["out_ref"]
    assert abs(out[0, 1] - want) < 1e-15
    mask = np.ones_like(out, bool)
    mask[0, 1] = False
    assert np.all(out[mask] == 0.0)
    assert res["out_bf16"][0, 1] == int(ex["out_bf16_0_1_bits"], 16)
    assert bf16_to_f64(res["out_bf16"])[0, 1] == ex["out_bf16_0_1_value"]


def test_worked_example_b(orc):
    g, inp, res = run_golden(orc, "worked_example_b.json")
    ex = g["expected"]
    np.testing.assert_array_equal(res["topk_ids"], ex["topk_ids"])
    l = float(np.float32(math.log(3.0)))
    s1, s0 = 1.0 / (1.0 + math.exp(-l)), 0.5
    wb = [s1 / (s0 + s1), s0 / (s0 + s1)]
    np.testing.assert_allclose(res["topk_w"][0], wb, rtol=1e-15)
    assert abs(wb[0] - 0.6) < 1e-8
    y0 = 0.5 * 7.0 / (1.0 + math.exp(-7.0)) * 1.0
    y1 = 1.0 * (-1.0) / (1.0 + math.exp(1.0)) * 3.0
    want = wb[0] * y1 + wb[1] * y0
    assert abs(want - ex["out_ref_0_1_value"]) < 1e-14
    assert abs(res["out_ref"][0, 1] - want) < 1e-15
    assert np.count_nonzero(res["out_ref"]) == 1
    assert res["out_bf16"][0, 1] == int(ex["out_bf16_0_1_bits"], 16)


@pytest.mark.parametrize("H,I,clamp", [(64, 32, 0.0), (96, 160, 0.0), (256, 128, 3.0)])
def test_single_expert_is_dense_swiglu_mlp(orc, H, I, clamp):
    T = 5
    rng = np.random.default_rng(H + I)
    x = moe_synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    w = moe_synth.make_weights(1, H, I, seed=H * 7 + I)
    ids = np.zeros((T, 1), np.int32)
    wt = np.ones((T, 1))
    res = orc.mxfp4_ffn(x, w["w13_q"], w["w13_s"], w["w2_q"], w["w2_s"], ids, wt, clamp)
    X = torch.from_numpy(bf16_to_f64(x))
    W13 = torch.from_numpy(dequant(w["w13_q"][0], w["w13_s"][0]))
    W2 = torch.from_numpy(dequant(w["w2_q"][0], w["w2_s"][0]))
    gate = X @ W13[:I].T
    up = X @ W13[I:].T
    if clamp > 0:
        gate = gate.clamp(-clamp, clamp)
        up = up.clamp(-clamp, clamp)
    ref = (torch.nn.functional.silu(gate) * up) @ W2.T
    np.testing.assert_allclose(res["out_ref"], ref.numpy(), rtol=1e-12, atol=1e-12 * float(ref.abs().max()))


@pytest.mark.parametrize("T,H,I,E,k,score_fn,clamp,seed", [
    (4, 256, 128, 8, 2, 0, 0.0, 0),
    (3, 64, 96, 5, 5, 0, 0.0, 1),
    (6, 128, 64, 8, 3, 1, 7.0, 2),
    (2, 32, 32, 3, 1, 1, 0.0, 3),
    (7, 96, 32, 16, 4, 0, 2.5, 4),
])
def test_matches_numpy_bruteforce(orc, T, H, I, E, k, score_fn, clamp, seed):
    cfg, inp = moe_synth.small_case(T, H, I, E, k, seed, score_fn=score_fn, clamp=clamp)
    ids, w = orc.route_topk(inp["logits"], k, score_fn)
    res = orc.mxfp4_ffn(inp["x"], inp["w13_q"], inp["w13_s"], inp["w2_q"], inp["w2_s"], ids, w, clamp)
    ref = numpy_bruteforce_ffn(inp["x"], inp["w13_q"], inp["w13_s"], inp["w2_q"], inp["w2_s"], ids, w,
                               clamp)
    np.testing.assert_allclose(res["out_ref"], ref, rtol=1e-11, atol=1e-11 * float(np.abs(ref).max()))


def test_tiny_config_matches_numpy_bruteforce(orc):
    cfg = moe_synth.CONFIGS["tiny"]
    inp = moe_synth.make_inputs(cfg)
    res = orc.moe_layer(inp["logits"], inp["x"], inp["w13_q"], inp["w13_s"], inp["w2_q"], inp["w2_s"],
                        cfg.k, cfg.score_fn, cfg.renorm, cfg.clamp)
    ref = numpy_bruteforce_ffn(inp["x"], inp["w13_q"], inp["w13_s"], inp["w2_q"], inp["w2_s"],
                               res["topk_ids"], res["topk_w"], cfg.clamp)
    np.testing.assert_allclose(res["out_ref"], ref, rtol=1e-11, atol=1e-11 * float(np.abs(ref).max()))


def _small(seed=11, clamp=0.0, score_fn=0):
    return moe_synth.small_case(5, 128, 64, 6, 3, seed, score_fn=score_fn, clamp=clamp)


def test_w2_scale_plus_one_doubles_output_exactly(orc):
    cfg, inp = _small()
    ids, w = orc.route_topk(inp["logits"], cfg.k)
    a = orc.mxfp4_ffn(inp["x"], inp["w13_q"], inp["w13_s"], inp["w2_q"], inp["w2_s"], ids, w)
    b = orc.mxfp4_ffn(inp["x"], inp["w13_q"], inp["w13_s"], inp["w2_q"], inp["w2_s"] + 1, ids, w)
    np.testing.assert_array_equal(b["out_ref"], 2.0 * a["out_ref"])


def test_up_scale_plus_one_doubles_output_exactly(orc):
    cfg, inp = _small()
    ids, w = orc.route_topk(inp["logits"], cfg.k)
    s = inp["w13_s"].copy()
    I = cfg.I
    s[:, I:, :] += 1
    a = orc.mxfp4_ffn(inp["x"], inp["w13_q"], inp["w13_s"], inp["w2_q"], inp["w2_s"], ids, w)
    b = orc.mxfp4_ffn(inp["x"], inp["w13_q"], s, inp["w2_q"], inp["w2_s"], ids, w)
    np.testing.assert_array_equal(b["out_ref"], 2.0 * a["out_ref"])


def test_gate_scale_change_is_not_linear(orc):
    # doubling the gate doubles silu's argument: the output must NOT simply double
    cfg, inp = _small()
    ids, w = orc.route_topk(inp["logits"], cfg.k)
    s = inp["w13_s"].copy()
    s[:, : cfg.I, :] += 1
    a = orc.mxfp4_ffn(inp["x"], inp["w13_q"], inp["w13_s"], inp["w2_q"], inp["w2_s"], ids, w)
    b = orc.mxfp4_ffn(inp["x"], inp["w13_q"], s, inp["w2_q"], inp["w2_s"], ids, w)
    assert not np.allclose(b["out_ref"], 2.0 * a["out_ref"])


def test_expert_relabelling_invariance(orc):
    cfg, inp = _small(seed=12)
    base = orc.moe_layer(inp["logits"], inp["x"], inp["w13_q"], inp["w13_s"], inp["w2_q"], inp["w2_s"],
                         cfg.k)
    perm = np.random.default_rng(0).permutation(cfg.E)  # new label of old expert e is perm[e]
    inv = np.argsort(perm)
    lg = inp["logits"][:, inv]
    res = orc.moe_layer(lg, inp["x"], inp["w13_q"][inv], inp["w13_s"][inv], inp["w2_q"][inv],
                        inp["w2_s"][inv], cfg.k)
    np.testing.assert_array_equal(res["topk_ids"], perm[base["topk_ids"]])
    # the softmax denominator is summed in the permuted label order, so only rounding may differ
    np.testing.assert_allclose(res["out_ref"], base["out_ref"], rtol=1e-13,
                               atol=1e-13 * float(np.abs(base["out_ref"]).max()))


def test_token_permutation_equivariance(orc):
    cfg, inp = _small(seed=13, clamp=1.5, score_fn=1)
    base = orc.moe_layer(inp["logits"], inp["x"], inp["w13_q"], inp["w13_s"], inp["w2_q"], inp["w2_s"],
                         cfg.k, 1, True, 1.5)
    perm = np.random.default_rng(1).permutation(cfg.T)
    res = orc.moe_layer(inp["logits"][perm], inp["x"][perm], inp["w13_q"], inp["w13_s"], inp["w2_q"],
                        inp["w2_s"], cfg.k, 1, True, 1.5)
    np.testing.assert_array_equal(res["out_ref"], base["out_ref"][perm])


def test_clamp_limits_gate_and_up(orc):
    # one expert, identity-like weights: gate = up = x[0] scaled; clamp must bound both
    H = I = 32
    x = np.zeros((1, H), np.float32)
    x[0, 0] = 5.0
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    w13_q = np.zeros((1, 2 * I, H // 2), np.uint8)
    w13_s = np.full((1, 2 * I, H // 32), 127, np.uint8)
    w2_q = np.zeros((1, H, I // 2), np.uint8)
    w2_s = np.full((1, H, I // 32), 127, np.uint8)
    w13_q[0, 0, 0] = 0x02  # gate row 0, element 0 = +1
    w13_q[0, I, 0] = 0x0A  # up row 0, element 0 = -1
    w2_q[0, 0, 0] = 0x02  # y[0] = h[0]
    ids = np.zeros((1, 1), np.int32)
    w = np.ones((1, 1))
    free = orc.mxfp4_ffn(xb, w13_q, w13_s, w2_q, w2_s, ids, w, 0.0)["out_ref"][0, 0]
    cl = orc.mxfp4_ffn(xb, w13_q, w13_s, w2_q, w2_s, ids, w, 2.0)["out_ref"][0, 0]
    assert abs(free - (5.0 / (1 + math.exp(-5.0)) * -5.0)) < 1e-14
    assert abs(cl - (2.0 / (1 + math.exp(-2.0)) * -2.0)) < 1e-14


def test_bf16_output_is_rounded_reference(orc):
    cfg, inp = _small(seed=14)
    ids, w = orc.route_topk(inp["logits"], cfg.k)
    res = orc.mxfp4_ffn(inp["x"], inp["w13_q"], inp["w13_s"], inp["w2_q"], inp["w2_s"], ids, w)
    # the oracle rounds the fp64 value once; torch rounds the fp32 value: they agree unless the
    # fp32 rounding itself lands on a bfloat16 tie, which random data essentially never does
    tb = torch.from_numpy(res["out_ref"]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.mean(tb == res["out_bf16"]) > 0.999


def test_thread_count_does_not_change_results(orc):
    cfg, inp = _small(seed=15)
    ids, w = orc.route_topk(inp["logits"], cfg.k)
    a = orc.mxfp4_ffn(inp["x"], inp["w13_q"], inp["w13_s"], inp["w2_q"], inp["w2_s"], ids, w, nthreads=1)
    b = orc.mxfp4_ffn(inp["x"], inp["w13_q"], inp["w13_s"], inp["w2_q"], inp["w2_s"], ids, w, nthreads=4)
    np.testing.assert_array_equal(a["out_ref"], b["out_ref"])


def test_empty_batch(orc):
    w = moe_synth.make_weights(2, 32, 32, seed=0)
    res = orc.mxfp4_ffn(np.zeros((0, 32), np.uint16), w["w13_q"], w["w13_s"], w["w2_q"], w["w2_s"],
                        np.zeros((0, 1), np.int32), np.zeros((0, 1)))
    assert res["out_ref"].shape == (0, 32)
