"""moe_layer_from_logits: bitwise the routing, grouping and FFN launches it stands for
(moe_route_topk + moe_group_tokens + moe_mxfp4_ffn with the same flags), on the decode configs and on
ragged shapes, both where the routing runs inside the gate_up launch and where it does not; the fp64
oracle on decode_m8; HIP-graph replay."""
import dataclasses

import numpy as np
import pytest
import torch

import moe_synth
from _gpu import assert_output_parity, dev, out_bits, run_layer, weights_to_device, x_to_device

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("mxfp4_mixture_experts_amd")


def from_logits(inp, cfg, flags, w):
    x = x_to_device(inp["x"])
    T = x.shape[0]
    ids = torch.full((T, cfg.k), -7, dtype=torch.int32, device="cuda")
    tw = torch.full((T, cfg.k), -7.0, dtype=torch.float32, device="cuda")
    out = moe.layer_from_logits(dev(inp["logits"]), x, w, cfg.k, cfg.score_fn, cfg.renorm, cfg.clamp, flags,
                                ids=ids, weights=tw)
    torch.cuda.synchronize()
    return out_bits(out), ids.cpu().numpy(), tw.cpu().numpy()


def check_same(inp, cfg, flags, routed):
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    assert moe.layer_from_logits_routed(T, H, I, E, k, flags) == routed
    w = weights_to_device(inp)
    ref = run_layer(inp, k, cfg.score_fn, cfg.clamp, flags, w=w, renorm=cfg.renorm)
    print(f"layer from logits T={T} H={H} I={I} E={E} k={k} flags={flags} routed={routed}", flush=True)
    out, ids, tw = from_logits(inp, cfg, flags, w)
    np.testing.assert_array_equal(ids, ref["topk_ids"])
    np.testing.assert_array_equal(tw.view(np.uint32), ref["topk_w"].view(np.uint32))
    np.testing.assert_array_equal(out, ref["out_bf16"])
    return out


@pytest.mark.parametrize("name", ["tiny", "decode_c1", "decode_m2", "decode_m8"])
def test_decode_configs_routed(name):
    cfg = moe_synth.CONFIGS[name]
    inp = moe_synth.make_inputs(cfg)
    for flags in (0, moe.SEPARATE_COMBINE, moe.FORCE_SMALL_M):
        check_same(inp, cfg, flags, True)
    check_same(inp, cfg, moe.UNFUSED_GATE_UP, False)  # the separate routing launches


SHAPES = [
    # T, H, I, E, k, score_fn, renorm, clamp, seed, routed
    (3, 256, 96, 9, 4, 1, True, 7.0, 1, True),        # sigmoid, clamp, ragged I
    (8, 2048, 256, 64, 8, 0, True, 0.0, 2, True),     # 64 pairs: the most the routed variant takes
    (5, 4096, 512, 256, 8, 0, True, 0.0, 3, True),    # two blocks per lane, 40 pairs over 256 experts
    (7, 1024, 544, 12, 5, 1, False, 3.0, 4, True),    # 35 pairs over 12 experts, no renormalisation
    (4, 512, 256, 100, 6, 0, False, 0.0, 5, True),    # 100 experts: two per lane in the top-k
    (8, 4096, 256, 8, 8, 0, True, 0.0, 6, True),      # every token on every expert (8 rows each)
    (1, 96, 160, 6, 1, 0, True, 0.0, 7, False),       # 3 blocks per lane: not the routed variant
    (2, 7168, 256, 16, 2, 0, True, 0.0, 8, False),    # 7 blocks per lane
    (12, 1024, 544, 12, 5, 1, True, 3.0, 9, False),   # 12 tokens: an expert may take the MFMA kernels
    (17, 512, 256, 16, 2, 0, True, 0.0, 10, False),
]


@pytest.mark.parametrize("case", SHAPES, ids=lambda c: "T%d_H%d_I%d_E%d_k%d" % c[:5])
def test_shapes(case):
    T, H, I, E, k, fn, renorm, clamp, seed, routed = case
    cfg, inp = moe_synth.small_case(T, H, I, E, k, seed, score_fn=fn, clamp=clamp)
    check_same(inp, dataclasses.replace(cfg, renorm=renorm), 0, routed)


def test_decode_m8_oracle(orc):
    cfg = moe_synth.CONFIGS["decode_m8"]
    inp = moe_synth.make_inputs(cfg)
    ref = orc.moe_layer(inp["logits"], inp["x"], inp["w13_q"], inp["w13_s"], inp["w2_q"], inp["w2_s"], cfg.k,
                        cfg.score_fn, cfg.renorm, cfg.clamp)
    out, ids, _ = from_logits(inp, cfg, 0, weights_to_device(inp))
    np.testing.assert_array_equal(ids, ref["topk_ids"])
    assert_output_parity(out, ref["out_ref"], "layer_from_logits decode_m8")


def test_graph_replay():
    """Captured in a HIP graph: every replay (with eager work between) equals the eager call."""
    cfg = moe_synth.CONFIGS["decode_m2"]
    inp = moe_synth.make_inputs(cfg)
    w = weights_to_device(inp)
    x = x_to_device(inp["x"])
    logits = dev(inp["logits"])
    T = x.shape[0]
    out = torch.empty((T, cfg.H), dtype=torch.bfloat16, device="cuda")
    ws = moe.layer_from_logits_workspace(T, cfg.H, cfg.I, cfg.E, cfg.k)
    moe.layer_from_logits(logits, x, w, cfg.k, cfg.score_fn, cfg.renorm, cfg.clamp, out=out, workspace=ws)
    torch.cuda.synchronize()
    eager = out_bits(out).copy()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        moe.layer_from_logits(logits, x, w, cfg.k, cfg.score_fn, cfg.renorm, cfg.clamp, out=out, workspace=ws,
                              stream=s)
    for rep in range(3):
        out.zero_()
        ws.fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"graph replay {rep}", flush=True)
        np.testing.assert_array_equal(out_bits(out), eager)
