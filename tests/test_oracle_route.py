"""Pins for the oracle's router: brute-force ranking, library softmax/sigmoid, invariants."""
import numpy as np
import pytest
from scipy.special import expit, softmax


def brute_topk(logits, k):
    T, E = logits.shape
    return np.array([sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k] for t in range(T)],
                    np.int32).reshape(T, k)


@pytest.mark.parametrize("E,k", [(8, 2), (7, 3), (64, 8), (65, 8), (128, 8), (256, 8), (512, 16),
                                 (5, 5), (1, 1)])
def test_ids_match_bruteforce_sort(orc, E, k):
    rng = np.random.default_rng(E * 100 + k)
    logits = rng.standard_normal((37, E)).astype(np.float32)
    ids, w = orc.route_topk(logits, k)
    np.testing.assert_array_equal(ids, brute_topk(logits, k))


def test_ties_go_to_lower_index(orc):
    logits = np.zeros((3, 10), np.float32)
    logits[1, [2, 7]] = 1.0
    logits[2, :] = -0.0
    logits[2, 4] = 0.0
    ids, w = orc.route_topk(logits, 4)
    np.testing.assert_array_equal(ids[0], [0, 1, 2, 3])
    np.testing.assert_array_equal(ids[1], [2, 7, 0, 1])
    np.testing.assert_array_equal(ids[2], [0, 1, 2, 3])  # -0 == +0: index order decides
    np.testing.assert_allclose(w[0], 0.25, rtol=0, atol=1e-15)


def test_softmax_renorm_invariants(orc):
    rng = np.random.default_rng(3)
    logits = (rng.standard_normal((200, 256)) * 3).astype(np.float32)
    ids, w = orc.route_topk(logits, 8)
    assert np.all(np.abs(w.sum(1) - 1.0) < 1e-14)
    assert np.all(np.diff(w, axis=1) <= 0)
    for t in range(200):
        assert len(set(ids[t].tolist())) == 8


def test_softmax_k_equals_E_is_plain_softmax(orc):
    rng = np.random.default_rng(4)
    logits = rng.standard_normal((20, 16)).astype(np.float32)
    ids, w = orc.route_topk(logits, 16)
    ref = softmax(logits.astype(np.float64), axis=1)
    got = np.zeros_like(ref)
    np.put_along_axis(got, ids.astype(np.int64), w, axis=1)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=0)


def test_softmax_without_renorm_is_full_softmax_probability(orc):
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((20, 64)).astype(np.float32)
    ids, w = orc.route_topk(logits, 8, score_fn=0, renorm=False)
    ref = softmax(logits.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(ref, ids.astype(np.int64), 1), rtol=1e-13)
    assert np.all(w.sum(1) < 1.0)


def test_sigmoid_scores(orc):
    rng = np.random.default_rng(6)
    logits = rng.standard_normal((20, 256)).astype(np.float32)
    ids, w = orc.route_topk(logits, 8, score_fn=1, renorm=False)
    np.testing.assert_array_equal(ids, brute_topk(logits, 8))
    np.testing.assert_allclose(w, expit(np.take_along_axis(logits, ids.astype(np.int64), 1)
                                        .astype(np.float64)), rtol=1e-14)
    ids2, w2 = orc.route_topk(logits, 8, score_fn=1, renorm=True)
    np.testing.assert_array_equal(ids2, ids)
    assert np.all(np.abs(w2.sum(1) - 1.0) < 1e-14)
    np.testing.assert_allclose(w2 * w.sum(1, keepdims=True), w, rtol=1e-14)


def test_k1_weight_is_one(orc):
    rng = np.random.default_rng(8)
    logits = rng.standard_normal((10, 33)).astype(np.float32)
    for fn in (0, 1):
        ids, w = orc.route_topk(logits, 1, score_fn=fn, renorm=True)
        np.testing.assert_array_equal(ids[:, 0], logits.argmax(1))
        assert np.all(w == 1.0)


def test_empty_batch(orc):
    ids, w = orc.route_topk(np.zeros((0, 8), np.float32), 2)
    assert ids.shape == (0, 2) and w.shape == (0, 2)
