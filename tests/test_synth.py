"""The seeded input generator: shapes, determinism and the stated value distributions."""
import numpy as np

import moe_synth


def test_shapes_and_determinism():
    cfg = moe_synth.CONFIGS["tiny"]
    a = moe_synth.make_inputs(cfg)
    b = moe_synth.make_inputs(cfg)
    assert a["logits"].shape == (4, 8) and a["x"].shape == (4, 256)
    assert a["w13_q"].shape == (8, 256, 128) and a["w13_s"].shape == (8, 256, 8)
    assert a["w2_q"].shape == (8, 256, 64) and a["w2_s"].shape == (8, 256, 4)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])


def test_scale_and_code_distributions():
    cfg = moe_synth.CONFIGS["tiny"]
    a = moe_synth.make_inputs(cfg)
    assert a["w13_s"].min() == 120 and a["w13_s"].max() == 124
    lo = a["w13_q"] & 0xF
    hi = a["w13_q"] >> 4
    for nib in (lo, hi):
        counts = np.bincount(nib.reshape(-1), minlength=16)
        assert counts.min() > 0.8 * nib.size / 16


def test_bf16_rounding_of_x():
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5], np.float32)
    np.testing.assert_array_equal(moe_synth.f32_to_bf16_bits(v), [0x3F80, 0x3F80, 0x3F82, 0xC020])


def test_uniform_and_zipf_logits():
    m2 = moe_synth.make_inputs(moe_synth.CONFIGS["decode_m2"], weights=False)
    assert m2["logits"].min() >= -1.0 and m2["logits"].max() < 1.0
    z = moe_synth.make_inputs(moe_synth.CONFIGS["medium_zipf"], weights=False)
    assert z["logits"].shape == (256, 256)
    bias = moe_synth.zipf_bias(256, z["zipf_rank"])
    # the most popular expert (rank 1) gets the largest bias
    assert np.argmax(bias) == int(np.argmin(z["zipf_rank"]))
