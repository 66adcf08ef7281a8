"""GPU parity of the whole layer on MXFP4 scale bytes far from the narrow band of the other tests.

The other parity tests draw every E8M0 byte from [120, 124]. Here, against the fp64 oracle, with
the bar of tests/_gpu.py and through every kernel family (weight-streaming, row-tile MFMA, dense
MFMA from 256 rows per expert):
  - scale bytes uniform over a wide band [96, 160] and over a realistic one [112, 136];
  - down and gate/up rows holding one block 40 below the row's largest byte (outside the 36-step
    window in which the dense down GEMM decodes its weights exactly);
  - the ends of the exactly decoded range, bytes 2 and 252, with activations that offset them so
    that products stay ordinary numbers (moe_synth.extreme_scale_case), and h varying over 2^120
    across the blocks of a row on the streaming and row-tile paths.
The MXFP4 element format is the OCP Microscaling Formats (MX) v1.0 definition (E2M1 codes, E8M0
scales 2^(s - 127))."""
import numpy as np
import pytest

import moe_synth
from _gpu import assert_output_parity, run_layer, weights_to_device

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("mxfp4_mixture_experts_amd")

FLAGS = {"default": 0, "small": moe.FORCE_SMALL_M, "large": moe.FORCE_LARGE_M}


def check(orc, cfg, inp, flag_names):
    ref = orc.moe_layer(inp["logits"], inp["x"], inp["w13_q"], inp["w13_s"], inp["w2_q"], inp["w2_s"],
                        cfg.k, cfg.score_fn, cfg.renorm, cfg.clamp)
    # the inputs keep the exact layer inside the bfloat16 range (a case that did not would test
    # overflow, not the decode)
    assert np.abs(ref["out_ref"]).max() < 2.0 ** 127
    w = weights_to_device(inp)
    for fname in flag_names:
        print(f"scales {cfg.name} flags={fname}", flush=True)
        g = run_layer(inp, cfg.k, cfg.score_fn, cfg.clamp, FLAGS[fname], w=w, renorm=cfg.renorm)
        np.testing.assert_array_equal(g["sorted_pair"], ref["sorted_pair"])
        assert_output_parity(g["out_bf16"], ref["out_ref"], f"{cfg.name}/{fname}")


# T, H, I, E, k, seed, flag sets (the 520-token cases give experts of >= 256 rows: dense kernels)
SHAPES = [
    (5, 256, 128, 6, 3, 41, ("default", "small", "large")),
    (40, 512, 256, 4, 2, 42, ("default", "small", "large")),
    (520, 256, 128, 2, 1, 43, ("default", "large")),
]


@pytest.mark.parametrize("band", [(96, 160), (112, 136)], ids=lambda b: "s%d-%d" % b)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda c: "T%d_H%d_I%d_E%d_k%d" % c[:5])
def test_scale_band(orc, band, shape):
    T, H, I, E, k, seed, flags = shape
    cfg, inp = moe_synth.small_case(T, H, I, E, k, seed, scale_lo=band[0], scale_hi=band[1])
    check(orc, cfg, inp, flags)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda c: "T%d_H%d_I%d_E%d_k%d" % c[:5])
def test_block_far_below_row_max(orc, shape):
    """One block per weight row 40 steps below the row's largest byte (realistic band otherwise)."""
    T, H, I, E, k, seed, flags = shape
    cfg, inp = moe_synth.small_case(T, H, I, E, k, seed + 100, scale_lo=112, scale_hi=136)
    inp["w2_s"] = moe_synth.lower_one_block_per_row(inp["w2_s"], 40, seed)
    inp["w13_s"] = moe_synth.lower_one_block_per_row(inp["w13_s"], 40, seed + 1)
    assert int((inp["w2_s"].max(axis=2) - inp["w2_s"].min(axis=2)).min()) >= 37
    check(orc, cfg, inp, flags)


EXTREME = [
    # T, H, I, E, k, seed, offsets of h per I-block, flag sets
    (6, 512, 256, 4, 2, 7, (0, 20, -20, 100), ("default", "small", "large")),
    (40, 256, 256, 4, 2, 8, (0, 20, -20, 100), ("default", "small", "large")),
    # dense down: h of a row is carried as one fp16 row (full precision down to 2^-28 of the row's
    # largest value), so the per-block offsets of h span 20 here; the byte-252 down blocks meet h of
    # about 2^-19, which keeps their sums near 2^114
    (300, 256, 256, 2, 2, 9, (30, 10, 20, 30), ("default", "large")),
]


@pytest.mark.parametrize("case", EXTREME, ids=lambda c: "T%d_H%d_I%d_E%d_k%d" % c[:5])
def test_scale_bytes_2_and_252(orc, case):
    T, H, I, E, k, seed, lam, flags = case
    cfg, inp = moe_synth.extreme_scale_case(T, H, I, E, k, seed, lam=lam)
    for a in ("w13_s", "w2_s"):
        assert (inp[a] == 2).any() and (inp[a] == 252).any()
    check(orc, cfg, inp, flags)
