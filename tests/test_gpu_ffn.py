"""GPU parity of the whole layer (route -> group -> moe_mxfp4_ffn) against the fp64 oracle.

Small workloads are compared element by element on every output; the full-size decode workloads too
(the oracle finishes them in seconds); the T=256/1024 workloads on sampled tokens, whose outputs the
oracle computes one token at a time (a token's output depends only on its own row, ids and weights).
Every case also runs with the weight-streaming and the MFMA kernels forced, and the unfused gate/up
variant, on the same inputs."""
import numpy as np
import pytest
import torch

import moe_synth
from _gpu import assert_output_parity, dev, out_bits, run_layer, sample_tokens, weights_to_device, x_to_device

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("mxfp4_mixture_experts_amd")

FLAG_SETS = {"default": 0, "small": moe.FORCE_SMALL_M, "large": moe.FORCE_LARGE_M,
             "unfused": moe.UNFUSED_GATE_UP, "unfused_small": moe.UNFUSED_GATE_UP | moe.FORCE_SMALL_M,
             "separate": moe.SEPARATE_COMBINE, "separate_small": moe.SEPARATE_COMBINE | moe.FORCE_SMALL_M}
# pairs of flag sets whose outputs must be bitwise equal: only the launch structure differs
SAME_BITS = (("unfused", "default"), ("unfused_small", "small"), ("separate", "default"),
             ("separate_small", "small"))


def oracle_full(orc, inp, cfg):
    return orc.moe_layer(inp["logits"], inp["x"], inp["w13_q"], inp["w13_s"], inp["w2_q"], inp["w2_s"],
                         cfg.k, cfg.score_fn, cfg.renorm, cfg.clamp)


def check_full(orc, cfg, inp, flags_names=tuple(FLAG_SETS)):
    ref = oracle_full(orc, inp, cfg)
    w = weights_to_device(inp)
    outs = {}
    for fname in flags_names:
        print(f"ffn {cfg.name} T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k} flags={fname}", flush=True)
        g = run_layer(inp, cfg.k, cfg.score_fn, cfg.clamp, FLAG_SETS[fname], w=w, renorm=cfg.renorm)
        np.testing.assert_array_equal(g["topk_ids"], ref["topk_ids"])
        np.testing.assert_array_equal(g["sorted_pair"], ref["sorted_pair"])
        assert_output_parity(g["out_bf16"], ref["out_ref"], f"{cfg.name}/{fname}")
        outs[fname] = g["out_bf16"]
    for a, b in SAME_BITS:
        if a in outs and b in outs:
            np.testing.assert_array_equal(outs[a], outs[b], err_msg=f"{a} vs {b}")
    return outs


@pytest.mark.parametrize("name", ["tiny", "decode_c1", "decode_m2"])
def test_configs_full(orc, name):
    cfg = moe_synth.CONFIGS[name]
    check_full(orc, cfg, moe_synth.make_inputs(cfg))


def test_decode_m8_full(orc):
    cfg = moe_synth.CONFIGS["decode_m8"]
    check_full(orc, cfg, moe_synth.make_inputs(cfg), ("default", "large", "unfused"))


FOLD_CASES = [
    # T, H, I, E, k, ids of every token (None: routed by the logits): the combine folded into down
    (1, 96, 160, 6, 1, [2]),                      # one pair; 64-row output tiles, the last ragged
    (2, 4096, 2048, 8, 8, [0, 0, 1, 0, 2, 0, 0, 7]),  # mixed multiplicities, 16 pairs
    (4, 256, 8192, 3, 2, None),                   # 4 blocks per lane, 8 pairs, h 139 KB in LDS
    (32, 224, 96, 40, 1, None),                   # 32 pairs (the most that fold), ragged tiles
    (16, 512, 256, 4, 2, [3, 3]),                 # 32 rows in one expert, tokens per pass 2
]


@pytest.mark.parametrize("case", FOLD_CASES, ids=lambda c: "T%d_H%d_I%d_E%d_k%d" % c[:5])
def test_folded_combine(orc, case):
    """Down with the combine folded in: the same bits as down + the separate combine launch, and the
    oracle's result within the tolerance."""
    T, H, I, E, k, row = case
    cfg, inp = moe_synth.small_case(T, H, I, E, k, 90 + T)
    if row is None:
        ids, wts = orc.route_topk(inp["logits"], k, cfg.score_fn, cfg.renorm)
    else:
        ids = np.tile(np.array(row, np.int32), (T, 1))
        wts = np.random.default_rng(T).uniform(0.05, 1.0, (T, k))
    wts = np.asarray(wts, np.float32).astype(np.float64)  # the weights the GPU is given, exactly
    ref = orc.mxfp4_ffn(inp["x"], inp["w13_q"], inp["w13_s"], inp["w2_q"], inp["w2_s"], ids, wts)
    assert moe.ffn_plan(T, H, I, E, k, moe.FORCE_SMALL_M)["fold_combine"] == 1
    assert moe.ffn_plan(T, H, I, E, k, moe.FORCE_SMALL_M | moe.SEPARATE_COMBINE)["fold_combine"] == 0
    w = weights_to_device(inp)
    outs = {}
    for fname in ("small", "separate_small"):
        print(f"folded combine T={T} H={H} I={I} E={E} k={k} flags={fname}", flush=True)
        g = run_layer(inp, k, 0, 0.0, FLAG_SETS[fname], w=w, ids=ids, topk_w=wts)
        assert_output_parity(g["out_bf16"], ref["out_ref"], f"fold T{T} I{I}/{fname}")
        outs[fname] = g["out_bf16"]
    np.testing.assert_array_equal(outs["small"], outs["separate_small"])


CASES = [
    # T, H, I, E, k, score_fn, clamp, seed: ragged shapes, blocks per lane 1..8, tails of every tile
    (5, 96, 160, 6, 3, 0, 0.0, 1),
    (3, 32, 32, 1, 1, 0, 0.0, 2),
    (7, 288, 96, 9, 4, 1, 7.0, 3),
    (2, 224, 736, 4, 2, 0, 0.0, 4),
    (9, 1024, 544, 12, 5, 1, 3.0, 5),
    (16, 512, 256, 16, 16, 0, 0.0, 6),
    (1, 7168, 256, 4, 2, 1, 7.0, 7),
    (40, 256, 128, 4, 2, 0, 0.0, 8),     # experts with ~20 rows each: both kernel families
    (130, 160, 96, 3, 2, 0, 0.0, 9),     # >64 rows per expert: several MFMA row tiles, ragged
    (33, 8192, 64, 5, 3, 0, 0.0, 10),
    (4, 128, 8192, 3, 2, 0, 0.0, 11),
    (6, 16384, 32, 2, 1, 0, 0.0, 12),   # 8 blocks per lane at the largest hidden size
]


DENSE_CASES = [
    # experts with >= 256 rows take the dense kernels (256-row tiles, operands staged in LDS)
    (600, 160, 96, 3, 2, 0, 0.0, 21),     # ~400 rows per expert: a full and a partial row tile;
                                          # 5 and 3 K-steps (odd: a padding step)
    (520, 256, 128, 2, 1, 1, 7.0, 22),    # ~260 rows: a 4-row second tile; sigmoid, clamp
    (512, 2048, 1024, 1, 1, 0, 0.0, 23),  # exactly two full tiles
    (300, 544, 320, 2, 2, 0, 0.0, 24),    # one expert >= 256, one below (row-tile kernels), columns
                                          # not a multiple of the column tiles
]


@pytest.mark.parametrize("case", DENSE_CASES, ids=lambda c: "T%d_H%d_I%d_E%d_k%d" % c[:5])
def test_dense_shapes(orc, case):
    T, H, I, E, k, fn, clamp, seed = case
    cfg, inp = moe_synth.small_case(T, H, I, E, k, seed, score_fn=fn, clamp=clamp)
    outs = check_full(orc, cfg, inp, ("default", "large", "unfused"))
    # both column tiles of the dense down GEMM: the tile decides which workgroup computes an output
    # column, not its arithmetic, so the bits are the same
    w = weights_to_device(inp)
    for cols in (256, 224):
        print(f"dense down with {cols}-column tiles", flush=True)
        g = run_layer(inp, cfg.k, cfg.score_fn, cfg.clamp, 0, w=w, renorm=cfg.renorm,
                      options=moe.ffn_options(dense_down_cols=cols))
        np.testing.assert_array_equal(g["out_bf16"], outs["default"])


def crafted_case(T, H, I, rows, seed):
    """k = 1, expert e receives exactly rows[e] tokens (logits one-hot on the chosen expert)."""
    E = len(rows)
    assert sum(rows) == T
    cfg, inp = moe_synth.small_case(T, H, I, E, 1, seed)
    owner = np.repeat(np.arange(E), rows)
    logits = np.zeros((T, E), np.float32)
    logits[np.arange(T), owner] = 1.0
    inp["logits"] = logits
    return cfg, inp


DENSE_EDGES = [
    # T, H, I, rows per expert: one row past a full tile; a 256-row dense expert next to a 255-row
    # row-tile expert; an output width that is a multiple of neither down column tile (480)
    (257, 96, 64, (257,), 31),
    (511, 160, 96, (256, 255), 32),
    (300, 480, 160, (300,), 33),
]


@pytest.mark.parametrize("case", DENSE_EDGES, ids=lambda c: "T%d_H%d_I%d_rows%s" % (c[0], c[1], c[2], "-".join(map(str, c[3]))))
def test_dense_edges(orc, case):
    T, H, I, rows, seed = case
    cfg, inp = crafted_case(T, H, I, rows, seed)
    ref = oracle_full(orc, inp, cfg)
    np.testing.assert_array_equal(ref["counts"], np.array(rows))
    w = weights_to_device(inp)
    outs = []
    for cols in (0, 256, 224):
        print(f"dense edge T={T} H={H} I={I} rows={rows} down cols={cols or 'auto'}", flush=True)
        g = run_layer(inp, cfg.k, cfg.score_fn, cfg.clamp, 0, w=w, renorm=cfg.renorm,
                      options=moe.ffn_options(dense_down_cols=cols))
        np.testing.assert_array_equal(g["sorted_pair"], ref["sorted_pair"])
        assert_output_parity(g["out_bf16"], ref["out_ref"], f"dense edge {rows} cols={cols}")
        outs.append(g["out_bf16"])
    for o in outs[1:]:
        np.testing.assert_array_equal(o, outs[0])


@pytest.mark.parametrize("case", CASES, ids=lambda c: "T%d_H%d_I%d_E%d_k%d" % c[:5])
def test_small_shapes(orc, case):
    T, H, I, E, k, fn, clamp, seed = case
    cfg, inp = moe_synth.small_case(T, H, I, E, k, seed, score_fn=fn, clamp=clamp)
    check_full(orc, cfg, inp)


def test_threshold_sweep_same_result(orc):
    """Every launch-table threshold gives an oracle-matching output on a mixed-M workload."""
    cfg, inp = moe_synth.small_case(48, 512, 256, 8, 3, 21)
    ref = oracle_full(orc, inp, cfg)
    w = weights_to_device(inp)
    for thr in (0, 1, 2, 4, 8, 16, 32, 1000):
        print(f"threshold {thr}", flush=True)
        g = run_layer(inp, cfg.k, cfg.score_fn, cfg.clamp, 0, w=w, options=moe.ffn_options(small_m_max=thr))
        assert_output_parity(g["out_bf16"], ref["out_ref"], f"thr={thr}")


@pytest.mark.parametrize("name", ["medium_zipf", "high_c4", "m1024"])
def test_large_configs_sampled(orc, name):
    cfg = moe_synth.CONFIGS[name]
    inp = moe_synth.make_inputs(cfg)
    ids, wts = orc.route_topk(inp["logits"], cfg.k, cfg.score_fn, cfg.renorm)
    grp = orc.group_tokens(ids, cfg.E)
    toks = sample_tokens(ids, grp, cfg.T, cfg.k)
    ref = orc.mxfp4_ffn(inp["x"][toks], inp["w13_q"], inp["w13_s"], inp["w2_q"], inp["w2_s"], ids[toks],
                        wts[toks], cfg.clamp)
    w = weights_to_device(inp)
    for fname in ("default", "large", "small"):
        print(f"ffn {name} flags={fname} sampled tokens {toks.tolist()}", flush=True)
        g = run_layer(inp, cfg.k, cfg.score_fn, cfg.clamp, FLAG_SETS[fname], w=w, renorm=cfg.renorm)
        np.testing.assert_array_equal(g["topk_ids"], ids)
        np.testing.assert_array_equal(g["counts"], grp["counts"])
        np.testing.assert_array_equal(g["sorted_pair"], grp["sorted_pair"])
        assert_output_parity(g["out_bf16"][toks], ref["out_ref"], f"{name}/{fname} ({len(toks)} tokens)")


DUP_IDS = [
    # T, H, I, E, k, ids of every token: repeated ids put several pairs of one token in one expert
    (8, 4096, 2048, 8, 8, [0] * 8),                   # one expert with all 64 rows
    (2, 4096, 2048, 8, 8, [0] * 8),                   # 16 rows: all of h fits the LDS (staged down)
    (8, 1024, 512, 8, 8, [0, 0, 0, 1, 1, 2, 4, 0]),   # mixed multiplicities
    (8, 4096, 2048, 8, 8, [0, 0, 0, 0, 1, 2, 3, 4]),  # h too big for LDS: workgroups within experts 1-4
                                                      # stage their rows, those in expert 0 (32 rows,
                                                      # 256 KB) read them from L2
    (300, 256, 128, 3, 2, [1, 1]),                     # 600 rows in one expert: dense kernels
]


@pytest.mark.parametrize("case", DUP_IDS, ids=lambda c: "T%d_H%d_I%d_E%d_k%d" % c[:5])
def test_duplicate_ids(orc, case):
    """The grouping accepts ids repeated within a token; every kernel family handles the expert
    that then holds more rows than there are tokens."""
    T, H, I, E, k, row = case
    cfg, inp = moe_synth.small_case(T, H, I, E, k, 50 + T)
    ids = np.tile(np.array(row, np.int32), (T, 1))
    wts = np.full((T, k), 1.0 / k)
    ref = orc.mxfp4_ffn(inp["x"], inp["w13_q"], inp["w13_s"], inp["w2_q"], inp["w2_s"], ids, wts)
    w = weights_to_device(inp)
    for fname in ("default", "small", "large"):
        print(f"duplicate ids T={T} H={H} I={I} E={E} k={k} flags={fname}", flush=True)
        g = run_layer(inp, k, 0, 0.0, FLAG_SETS[fname], w=w, ids=ids)
        np.testing.assert_array_equal(g["counts"], np.bincount(ids.ravel(), minlength=E))
        assert_output_parity(g["out_bf16"], ref["out_ref"], f"dup ids T{T} I{I} {row}/{fname}")


def test_empty_batch():
    w = moe.Mxfp4Weights(*(torch.zeros(s, dtype=torch.uint8, device="cuda")
                           for s in [(2, 64, 16), (2, 64, 1), (2, 32, 16), (2, 32, 1)]))
    x = torch.zeros((0, 32), dtype=torch.bfloat16, device="cuda")
    ids, tw = moe.route_topk(torch.zeros((0, 2), device="cuda"), 1)
    grp = moe.group_tokens(ids, 2)
    out = moe.mxfp4_ffn(x, w, tw, grp)
    torch.cuda.synchronize()
    assert out.shape == (0, 32)
    assert int(grp.n_active.item()) == 0 and int(grp.counts.sum().item()) == 0


def test_binding_rejects_mismatched_shapes():
    """The binding checks shapes, dtypes and buffer sizes before any launch (MoeError)."""
    cfg, inp = moe_synth.small_case(4, 256, 128, 8, 2, 77)
    w = weights_to_device(inp)
    x = x_to_device(inp["x"])
    logits = dev(inp["logits"])
    layer = moe.MoELayer(w, 2, 4)
    ids, tw = moe.route_topk(logits, 2)
    grp = moe.group_tokens(ids, 8)
    bad = [
        lambda: layer.forward(x, dev(np.zeros((4, 9), np.float32))),       # logits wider than E
        lambda: layer.forward(x, dev(np.zeros((5, 8), np.float32))),       # more logits rows than tokens
        lambda: layer.forward(x[:, :128], logits),                          # hidden size
        lambda: layer.forward(torch.zeros((5, 256), dtype=torch.bfloat16, device="cuda"),
                              dev(np.zeros((5, 8), np.float32))),          # above capacity
        lambda: moe.mxfp4_ffn(x[:, :224], w, tw, grp),                      # x width != H
        lambda: moe.mxfp4_ffn(x.float(), w, tw, grp),                       # x dtype
        lambda: moe.mxfp4_ffn(x.t().contiguous().t(), w, tw, grp),          # x not contiguous
        lambda: moe.mxfp4_ffn(x, w, tw[:3], grp),                           # topk_w rows != T
        lambda: moe.mxfp4_ffn(x, w, tw, moe.Grouping.empty(4, 2, 4, "cuda")),  # grouping for E=4
        lambda: moe.mxfp4_ffn(x, w, tw, moe.Grouping.empty(2, 2, 8, "cuda")),  # grouping for P=4
        lambda: moe.mxfp4_ffn(x, w, tw, grp, workspace=torch.empty(16, dtype=torch.uint8, device="cuda")),
        lambda: moe.mxfp4_ffn(x, w, tw, grp, out=torch.empty((4, 128), dtype=torch.bfloat16, device="cuda")),
        lambda: moe.group_tokens(ids, 8, out=moe.Grouping.empty(4, 2, 4, "cuda")),
        lambda: moe.route_topk(logits, 2, ids=torch.empty((4, 3), dtype=torch.int32, device="cuda")),
    ]
    for i, f in enumerate(bad):
        print(f"binding check #{i}", flush=True)
        with pytest.raises(moe.MoeError):
            f()
    torch.cuda.synchronize()
