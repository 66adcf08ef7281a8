"""Pins for the oracle's token-to-expert grouping: brute-force stable sort and invariants."""
import numpy as np
import pytest


def check_group(g, ids, E):
    flat = ids.reshape(-1)
    P = flat.size
    np.testing.assert_array_equal(g["counts"], np.bincount(flat, minlength=E))
    np.testing.assert_array_equal(g["offsets"], np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    order = sorted(range(P), key=lambda p: (int(flat[p]), p))
    np.testing.assert_array_equal(g["sorted_pair"], order)
    inv = np.empty(P, np.int64)
    inv[np.array(order, np.int64)] = np.arange(P)
    np.testing.assert_array_equal(g["pair_pos"], inv)
    np.testing.assert_array_equal(g["active"], np.nonzero(np.bincount(flat, minlength=E))[0])
    assert int(g["n_active"][0]) == len(g["active"])
    assert int(g["counts"].sum()) == P and int(g["offsets"][-1]) == P


@pytest.mark.parametrize("T,k,E,seed", [(4, 2, 8, 0), (1, 8, 128, 1), (8, 8, 256, 2),
                                        (256, 8, 256, 3), (33, 3, 5, 4), (100, 1, 512, 5)])
def test_group_matches_bruteforce(orc, T, k, E, seed):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    check_group(orc.group_tokens(ids, E), ids, E)


def test_group_skewed_with_empty_experts(orc):
    rng = np.random.default_rng(9)
    E, k, T = 64, 4, 50
    ids = np.stack([np.sort(rng.choice(8, size=k, replace=False)) for _ in range(T)]).astype(np.int32)
    g = orc.group_tokens(ids, E)
    check_group(g, ids, E)
    assert int(g["n_active"][0]) <= 8


def test_group_from_router_output(orc):
    rng = np.random.default_rng(10)
    logits = rng.standard_normal((40, 32)).astype(np.float32)
    ids, _ = orc.route_topk(logits, 4)
    check_group(orc.group_tokens(ids, 32), ids, 32)


def test_group_empty(orc):
    g = orc.group_tokens(np.zeros((0, 2), np.int32), 8)
    assert int(g["n_active"][0]) == 0 and g["counts"].sum() == 0
    np.testing.assert_array_equal(g["offsets"], np.zeros(9))
