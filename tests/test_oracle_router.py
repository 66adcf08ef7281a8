"""Pins of the oracle's router logits (logits = x . W_router^T, bfloat16 operands, fp64 sum) against
values fixed by the definition rather than by the oracle: a hand-worked case, one-hot activation rows
(each logit is then one weight, exactly), and integer-valued operands whose products and sums are
exact, compared with exact integer arithmetic."""
import numpy as np
import pytest

from _util import bf16_to_f64


def bf16(v):
    return (np.asarray(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_hand_worked(orc):
    # [1, 2, -0.5] . [3, 4, 2] = 10;  [1, 2, -0.5] . [0.5, -1, 8] = -5.5
    got = orc.router_logits(bf16([[1.0, 2.0, -0.5]]), bf16([[3, 4, 2], [0.5, -1, 8]]))
    np.testing.assert_array_equal(got, [[10.0, -5.5]])


@pytest.mark.parametrize("H,E", [(1, 1), (7, 3), (96, 40)])
def test_one_hot_rows_pick_weights(orc, H, E):
    """x = identity rows: logit (t, e) is exactly weight (e, t) (a transposed operand would fail)."""
    rng = np.random.default_rng(H * 100 + E)
    w = bf16(rng.standard_normal((E, H)).astype(np.float32))
    x = bf16(np.eye(H, dtype=np.float32))
    np.testing.assert_array_equal(orc.router_logits(x, w), bf16_to_f64(w).T)


@pytest.mark.parametrize("T,H,E,seed", [(1, 32, 8, 0), (5, 257, 13, 1), (9, 2048, 64, 2)])
def test_integer_operands_exact(orc, T, H, E, seed):
    """Integers in [-8, 8] are exact in bfloat16, and every partial sum stays far below 2^53, so the
    fp64 result must equal the integer matrix product."""
    rng = np.random.default_rng(seed)
    xi = rng.integers(-8, 9, size=(T, H))
    wi = rng.integers(-8, 9, size=(E, H))
    got = orc.router_logits(bf16(xi.astype(np.float32)), bf16(wi.astype(np.float32)))
    np.testing.assert_array_equal(got, (xi @ wi.T).astype(np.float64))


def test_thread_count_does_not_matter(orc):
    rng = np.random.default_rng(7)
    x = bf16(rng.standard_normal((6, 300)).astype(np.float32))
    w = bf16(rng.standard_normal((20, 300)).astype(np.float32))
    np.testing.assert_array_equal(orc.router_logits(x, w, nthreads=1), orc.router_logits(x, w, nthreads=4))
