"""The single-launch decode layer (moe_layer_decode): route, group, gate_up, down and combine in one
kernel. Against the fp64 oracle with the output bar of tests/_gpu.py; routing ids bitwise equal to
the separate router's and the oracle's; deterministic (bitwise equal over repeated calls, and under
HIP-graph replay); nothing written outside its workspace and output; no barrier wait gave up."""
import numpy as np
import pytest
import torch

import moe_synth
from _gpu import assert_output_parity, dev, out_bits, weight_rtol, weights_to_device, x_to_device

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("mxfp4_mixture_experts_amd")


def status_word(ws: torch.Tensor) -> int:
    """The workspace's count of barrier waits that gave up (bytes 8..11)."""
    return int(ws[8:12].cpu().numpy().view(np.uint32)[0])


def check_layer(orc, cfg, inp, label, repeats=3):
    ref = orc.moe_layer(inp["logits"], inp["x"], inp["w13_q"], inp["w13_s"], inp["w2_q"], inp["w2_s"],
                        cfg.k, cfg.score_fn, cfg.renorm, cfg.clamp)
    w = weights_to_device(inp)
    x = x_to_device(inp["x"])
    logits = dev(inp["logits"])
    ws = moe.layer_decode_workspace(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k)
    ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    tw = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda")
    first = None
    for r in range(repeats):
        print(f"layer_decode {label} T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k} call {r}", flush=True)
        out = moe.layer_decode(logits, x, w, cfg.k, cfg.score_fn, cfg.renorm, cfg.clamp, workspace=ws, ids=ids,
                               weights=tw)
        torch.cuda.synchronize()
        bits = out_bits(out)
        if first is None:
            first = bits
            np.testing.assert_array_equal(ids.cpu().numpy(), ref["topk_ids"])
            np.testing.assert_allclose(tw.cpu().numpy(), ref["topk_w"], rtol=weight_rtol(cfg.k), atol=0)
            # the same routing code as the separate router: bitwise equal ids and weights
            ids2, tw2 = moe.route_topk(logits, cfg.k, cfg.score_fn, cfg.renorm)
            np.testing.assert_array_equal(ids.cpu().numpy(), ids2.cpu().numpy())
            np.testing.assert_array_equal(tw.cpu().numpy(), tw2.cpu().numpy())
            assert_output_parity(bits, ref["out_ref"], f"layer_decode {label}")
        else:
            np.testing.assert_array_equal(bits, first)
    assert status_word(ws) == 0
    return first


@pytest.mark.parametrize("name", ["tiny", "decode_c1", "decode_m2", "decode_m8"])
def test_layer_configs(orc, name):
    cfg = moe_synth.CONFIGS[name]
    check_layer(orc, cfg, moe_synth.make_inputs(cfg), name)


SHAPES = [
    # T, H, I, E, k, score_fn, clamp, seed: gate_up blocks per lane 1..7, ragged I (in blocks of 32),
    # one expert, every expert active, more units than workgroups and fewer, k = 16, T = 16
    (1, 32, 32, 1, 1, 0, 0.0, 1),
    (5, 96, 160, 6, 3, 0, 0.0, 2),
    (7, 288, 96, 9, 4, 1, 7.0, 3),
    (3, 7168, 2048, 256, 8, 1, 7.0, 4),
    (16, 4096, 2048, 256, 8, 0, 0.0, 5),
    (16, 512, 256, 16, 16, 0, 0.0, 6),
    (9, 1024, 544, 12, 5, 1, 3.0, 7),
    (2, 224, 736, 4, 2, 0, 0.0, 8),
    (12, 2048, 4096, 32, 4, 0, 0.0, 9),
    (4, 16384, 64, 3, 2, 0, 0.0, 10),
]


@pytest.mark.parametrize("case", SHAPES, ids=lambda c: "T%d_H%d_I%d_E%d_k%d" % c[:5])
def test_layer_shapes(orc, case):
    T, H, I, E, k, fn, clamp, seed = case
    cfg, inp = moe_synth.small_case(T, H, I, E, k, seed, score_fn=fn, clamp=clamp)
    check_layer(orc, cfg, inp, cfg.name, repeats=2)


def test_layer_wide_scales(orc):
    cfg, inp = moe_synth.extreme_scale_case(6, 512, 256, 4, 2, 7)
    check_layer(orc, cfg, inp, "extreme scales", repeats=1)


def test_layer_graph_replay_and_guard():
    """One hipGraph of the launch replayed 5 times with eager calls between: every replay equals the
    eager result; guard bytes around the workspace tail and the output untouched."""
    cfg = moe_synth.CONFIGS["decode_m8"]
    inp = moe_synth.make_inputs(cfg)
    w = weights_to_device(inp)
    x = x_to_device(inp["x"])
    logits = dev(inp["logits"])
    need = moe.layer_decode_workspace_size(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k)
    guard = 1 << 16
    buf = torch.zeros(need + guard, dtype=torch.uint8, device="cuda")
    buf[need:] = 0xA5
    ws = buf[:need]
    out_buf = torch.full((cfg.T + 2, cfg.H), 7.0, dtype=torch.bfloat16, device="cuda")
    out = out_buf[1:cfg.T + 1]
    moe.layer_decode(logits, x, w, cfg.k, workspace=ws, out=out)
    torch.cuda.synchronize()
    eager = out_bits(out).copy()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        moe.layer_decode(logits, x, w, cfg.k, workspace=ws, out=out, stream=s)
    for i in range(5):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"layer_decode graph replay #{i}", flush=True)
        np.testing.assert_array_equal(out_bits(out), eager)
        moe.layer_decode(logits, x, w, cfg.k, workspace=ws, out=out)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out_bits(out), eager)
    assert torch.all(buf[need:] == 0xA5)
    assert torch.all(out_buf[0] == 7.0) and torch.all(out_buf[cfg.T + 1] == 7.0)
    assert status_word(ws) == 0


def test_moelayer_single_launch_matches_oracle(orc):
    cfg = moe_synth.CONFIGS["decode_m8"]
    inp = moe_synth.make_inputs(cfg)
    layer = moe.MoELayer(weights_to_device(inp), cfg.k, cfg.T, single_launch=True)
    ref = orc.moe_layer(inp["logits"], inp["x"], inp["w13_q"], inp["w13_s"], inp["w2_q"], inp["w2_s"], cfg.k)
    for T in (8, 3, 1):  # smaller batches through the same layer
        print(f"MoELayer single launch T={T}", flush=True)
        out = layer.forward(x_to_device(inp["x"][:T]), dev(inp["logits"][:T]))
        torch.cuda.synchronize()
        r = ref if T == cfg.T else orc.moe_layer(inp["logits"][:T], inp["x"][:T], inp["w13_q"], inp["w13_s"],
                                                  inp["w2_q"], inp["w2_s"], cfg.k)
        assert_output_parity(out_bits(out), r["out_ref"], f"MoELayer single launch T={T}")


def test_unsupported_shapes_rejected():
    assert moe.layer_decode_workspace_size(17, 4096, 2048, 256, 8) == 0   # T > 16
    assert moe.layer_decode_workspace_size(16, 4096, 2048, 256, 16) == 0  # 64 blocks per workgroup
    with pytest.raises(moe.MoeError):
        moe.layer_decode_workspace(17, 4096, 2048, 256, 8)
