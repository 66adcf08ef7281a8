"""GPU parity of the router (moe_route_topk), the grouping (moe_group_tokens) and their fused call
(moe_route_group) against the oracle:
ids, counts, offsets, permutation and active list bit-exact; routing weights within the fp32 bound."""
import numpy as np
import pytest
import torch

import moe_synth
from _gpu import dev, weight_rtol

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("mxfp4_mixture_experts_amd")


def gpu_route(logits, k, score_fn=0, renorm=True):
    ids, w = moe.route_topk(dev(logits), k, score_fn, renorm)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


def check_route(orc, logits, k, score_fn=0, renorm=True, label=""):
    print(f"route {label} T={logits.shape[0]} E={logits.shape[1]} k={k} fn={score_fn} renorm={renorm}",
          flush=True)
    ids, w = gpu_route(logits, k, score_fn, renorm)
    oids, ow = orc.route_topk(logits, k, score_fn, renorm)
    np.testing.assert_array_equal(ids, oids)
    n_terms = k if (renorm or score_fn == 1) else logits.shape[1]
    np.testing.assert_allclose(w, ow, rtol=weight_rtol(n_terms), atol=0)


@pytest.mark.parametrize("name", ["tiny", "decode_c1", "decode_m2", "decode_m8", "medium_zipf", "high_c4",
                                  "m1024"])
def test_route_configs(orc, name):
    cfg = moe_synth.CONFIGS[name]
    inp = moe_synth.make_inputs(cfg, weights=False)
    check_route(orc, inp["logits"], cfg.k, cfg.score_fn, cfg.renorm, name)


@pytest.mark.parametrize("E,k", [(1, 1), (7, 7), (64, 8), (65, 3), (128, 16), (300, 5), (512, 16), (512, 1)])
@pytest.mark.parametrize("score_fn,renorm", [(0, True), (0, False), (1, True), (1, False)])
def test_route_shapes(orc, E, k, score_fn, renorm):
    rng = np.random.default_rng(E * 31 + k)
    logits = (rng.standard_normal((45, E)) * 2).astype(np.float32)
    check_route(orc, logits, k, score_fn, renorm, "shapes")


def test_route_ties_and_signed_zero(orc):
    logits = np.zeros((4, 96), np.float32)
    logits[1, [5, 70, 33]] = 2.0
    logits[2, :] = -0.0
    logits[2, 50] = 0.0
    logits[3, ::2] = -1e30
    check_route(orc, logits, 6, 0, True, "ties")
    check_route(orc, logits, 6, 1, True, "ties-sigmoid")


def test_route_empty():
    ids, w = moe.route_topk(torch.zeros((0, 8), device="cuda"), 2)
    torch.cuda.synchronize()
    assert ids.shape == (0, 2)


def check_group(orc, ids, E, label=""):
    print(f"group {label} T={ids.shape[0]} k={ids.shape[1]} E={E}", flush=True)
    grp = moe.group_tokens(dev(ids.astype(np.int32)), E)
    torch.cuda.synchronize()
    ref = orc.group_tokens(ids, E)
    P = ids.size
    np.testing.assert_array_equal(grp.counts.cpu().numpy(), ref["counts"])
    np.testing.assert_array_equal(grp.offsets.cpu().numpy(), ref["offsets"])
    if P:
        np.testing.assert_array_equal(grp.sorted_pair[:P].cpu().numpy(), ref["sorted_pair"])
        np.testing.assert_array_equal(grp.pair_pos[:P].cpu().numpy(), ref["pair_pos"])
    n = int(grp.n_active.item())
    assert n == int(ref["n_active"][0])
    act = grp.active.cpu().numpy()
    np.testing.assert_array_equal(act[:n], ref["active"])
    assert np.all(act[n:] == -1)


@pytest.mark.parametrize("name", ["tiny", "decode_c1", "decode_m2", "decode_m8", "medium_zipf", "high_c4",
                                  "m1024"])
def test_group_configs(orc, name):
    cfg = moe_synth.CONFIGS[name]
    inp = moe_synth.make_inputs(cfg, weights=False)
    ids, _ = orc.route_topk(inp["logits"], cfg.k, cfg.score_fn)
    check_group(orc, ids, cfg.E, name)


@pytest.mark.parametrize("T,k,E,seed", [(1, 1, 1, 0), (3, 2, 5, 1), (64, 8, 256, 2), (1000, 16, 512, 3),
                                        (8192, 8, 256, 4), (4097, 3, 16, 5), (20000, 8, 512, 6),
                                        (1024, 2, 3, 12), (2049, 1, 7, 13), (1025, 2, 64, 14),
                                        (131072, 8, 64, 15), (1025, 1, 9, 19), (512, 2, 9, 20)])
def test_group_random(orc, T, k, E, seed):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    check_group(orc, ids, E, "random")


def test_group_skewed(orc):
    rng = np.random.default_rng(11)
    ids = np.stack([rng.choice(4, size=2, replace=False) for _ in range(3000)]).astype(np.int32)
    check_group(orc, ids, 512, "skewed")


@pytest.mark.parametrize("T,k,E,seed", [(3000, 4, 1, 16), (5000, 8, 8, 17), (700, 16, 3, 18)])
def test_group_repeated_ids(orc, T, k, E, seed):
    """ids drawn with repetition (an expert holds several pairs of one token), past the
    single-workgroup size; E = 1 puts every pair on one expert."""
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    check_group(orc, ids, E, "repeated")


def test_group_empty(orc):
    check_group(orc, np.zeros((0, 4), np.int32), 16, "empty")


@pytest.mark.parametrize("T,E,k,score_fn,renorm", [(1, 128, 8, 0, True), (8, 256, 8, 0, True), (2, 64, 1, 1, False),
                                                   (16, 512, 16, 1, True), (17, 300, 5, 0, False),
                                                   (64, 512, 16, 1, True),
                                                   (65, 256, 8, 0, True), (200, 64, 6, 1, True),
                                                   (0, 32, 4, 0, True)])
def test_route_group_matches_separate_calls(orc, T, E, k, score_fn, renorm):
    """moe_route_group (one launch for T <= 16, the two kernels above) equals route_topk followed by
    group_tokens bit for bit, and the oracle on ids and grouping."""
    print(f"route_group T={T} E={E} k={k} fn={score_fn} renorm={renorm}", flush=True)
    rng = np.random.default_rng(T * 1000 + E + k)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    lg = dev(logits) if T else torch.empty((0, E), dtype=torch.float32, device="cuda")
    ids_f, w_f, g_f = moe.route_group(lg, k, score_fn, renorm)
    ids_s, w_s = moe.route_topk(lg, k, score_fn, renorm)
    g_s = moe.group_tokens(ids_s, E)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids_f.cpu().numpy(), ids_s.cpu().numpy())
    np.testing.assert_array_equal(w_f.cpu().numpy().view(np.uint32), w_s.cpu().numpy().view(np.uint32))
    P = T * k
    for name in ("counts", "offsets", "active", "n_active"):
        np.testing.assert_array_equal(getattr(g_f, name).cpu().numpy(), getattr(g_s, name).cpu().numpy())
    for name in ("sorted_pair", "pair_pos"):
        np.testing.assert_array_equal(getattr(g_f, name)[:P].cpu().numpy(), getattr(g_s, name)[:P].cpu().numpy())
    if T:
        oids, _ = orc.route_topk(logits, k, score_fn, renorm)
        np.testing.assert_array_equal(ids_f.cpu().numpy(), oids)
        ref = orc.group_tokens(oids, E)
        np.testing.assert_array_equal(g_f.sorted_pair[:P].cpu().numpy(), ref["sorted_pair"])
