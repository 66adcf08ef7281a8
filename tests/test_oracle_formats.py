"""Pins for the oracle's scalar formats: E2M1, E8M0, element addressing and bfloat16 rounding."""
import math

import numpy as np
import pytest
import torch

from _util import E2M1_TABLE, dequant


def test_e2m1_all_codes_match_spec_table(orc):
    for code in range(16):
        v = orc.e2m1_value(code)
        mag = E2M1_TABLE[code & 7]
        assert abs(v) == mag, code
        assert math.copysign(1.0, v) == (-1.0 if code & 8 else 1.0), code


@pytest.mark.parametrize("s", [0, 1, 2, 100, 120, 121, 122, 123, 124, 126, 127, 128, 200, 254])
def test_e8m0_is_power_of_two(orc, s):
    assert orc.e8m0_value(s) == 2.0 ** (s - 127)


def test_e8m0_255_is_nan(orc):
    assert math.isnan(orc.e8m0_value(255))


def test_nibble_order_and_scale_blocks(orc):
    # one 64-element row: byte 0 = 0x21 -> element 0 = code 1 (0.5), element 1 = code 2 (1.0)
    q = np.zeros((2, 32), np.uint8)
    s = np.array([[127, 128], [126, 127]], np.uint8)
    q[0, 0] = 0x21
    q[0, 16] = 0x7F  # elements 32 (code 15 = -6) and 33 (code 7 = 6), in the second scale block (x2)
    q[1, 31] = 0x90  # row 1, elements 62 (code 0) and 63 (code 9 = -0.5), scale block 1 (x1)
    assert orc.mxfp4_element(q, s, 64, 0, 0) == 0.5
    assert orc.mxfp4_element(q, s, 64, 0, 1) == 1.0
    assert orc.mxfp4_element(q, s, 64, 0, 32) == -12.0
    assert orc.mxfp4_element(q, s, 64, 0, 33) == 12.0
    assert orc.mxfp4_element(q, s, 64, 1, 62) == 0.0
    assert orc.mxfp4_element(q, s, 64, 1, 63) == -0.5
    full = dequant(q, s)
    for n in range(2):
        for kk in range(64):
            assert orc.mxfp4_element(q, s, 64, n, kk) == full[n, kk]


def test_random_elements_match_table_dequant(orc):
    rng = np.random.default_rng(7)
    q = rng.integers(0, 256, size=(5, 48), dtype=np.uint8)
    s = rng.integers(1, 255, size=(5, 3), dtype=np.uint8)
    full = dequant(q, s)
    for n in range(5):
        for kk in range(96):
            assert orc.mxfp4_element(q, s, 96, n, kk) == full[n, kk]


def test_bf16_to_double_matches_torch(orc):
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 16, size=2000, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    for b, r in zip(bits, ref):
        v = orc.bf16_to_float(int(b))
        if math.isnan(r):
            assert math.isnan(v)
        else:
            assert v == r


def test_bf16_rounding_ties_to_even(orc):
    assert orc.float_to_bf16(1.0) == 0x3F80
    assert orc.float_to_bf16(1.0 + 2.0 ** -8) == 0x3F80  # halfway, even neighbour is 1.0
    assert orc.float_to_bf16(1.0 + 3 * 2.0 ** -8) == 0x3F82  # halfway, even neighbour is 1+2^-6
    assert orc.float_to_bf16(1.0 + 2.0 ** -8 + 2.0 ** -30) == 0x3F81  # just above halfway
    assert orc.float_to_bf16(-0.0) == 0x8000
    assert orc.float_to_bf16(float("inf")) == 0x7F80
    assert orc.float_to_bf16(3.5e38) == 0x7F80  # past the largest finite bfloat16
    assert orc.float_to_bf16(2.0 ** -133) == 0x0001  # smallest subnormal


def test_bf16_rounding_matches_torch_on_float32_values(orc):
    rng = np.random.default_rng(2)
    vals = np.concatenate([rng.standard_normal(3000).astype(np.float32),
                           (rng.standard_normal(500) * 1e-39).astype(np.float32),
                           (rng.standard_normal(500) * 1e30).astype(np.float32)])
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for v, r in zip(vals, ref):
        assert orc.float_to_bf16(float(v)) == int(r), float(v)
