"""Determinism and capture: repeated calls are bitwise identical, a HIP-graph replay of the whole
layer equals the eager result bitwise on every replay, and the workspace contract holds (nothing is
written past the queried size)."""
import numpy as np
import pytest
import torch

import moe_synth
from _gpu import out_bits, weights_to_device, x_to_device, dev

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("mxfp4_mixture_experts_amd")


@pytest.mark.parametrize("name,flags", [("decode_m8", 0), ("decode_m8", moe.FORCE_LARGE_M),
                                        ("tiny", moe.UNFUSED_GATE_UP)])
def test_repeat_bitwise(name, flags):
    cfg = moe_synth.CONFIGS[name]
    inp = moe_synth.make_inputs(cfg)
    layer = moe.MoELayer(weights_to_device(inp), cfg.k, cfg.T, cfg.score_fn, cfg.renorm, cfg.clamp, flags)
    x, lg = x_to_device(inp["x"]), dev(inp["logits"])
    first = out_bits(layer.forward(x, lg).clone())
    for i in range(10):
        print(f"repeat {name} flags={flags} #{i}", flush=True)
        np.testing.assert_array_equal(out_bits(layer.forward(x, lg)), first)


def test_graph_replay_equals_eager():
    cfg = moe_synth.CONFIGS["decode_m8"]
    inp = moe_synth.make_inputs(cfg)
    layer = moe.MoELayer(weights_to_device(inp), cfg.k, cfg.T, cfg.score_fn, cfg.renorm, cfg.clamp)
    x, lg = x_to_device(inp["x"]), dev(inp["logits"])
    eager = out_bits(layer.forward(x, lg).clone())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer.forward(x, lg)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = layer.forward(x, lg)
    for i in range(5):
        layer.out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"graph replay #{i}", flush=True)
        np.testing.assert_array_equal(out_bits(out), eager)
        # eager work between replays
        np.testing.assert_array_equal(out_bits(layer.forward(x, lg)), eager)


@pytest.mark.parametrize("T", [1, 2, 3, 8, 17, 64])
def test_workspace_guard(T):
    """The workspace is surrounded by a guard pattern that no call may touch, at every M."""
    cfg, inp = moe_synth.small_case(T, 512, 256, 16, 4, 100 + T)
    w = weights_to_device(inp)
    x, lg = x_to_device(inp["x"]), dev(inp["logits"])
    for flags in (0, moe.FORCE_LARGE_M, moe.UNFUSED_GATE_UP):
        need = moe.ffn_workspace_size(T, cfg.H, cfg.I, cfg.E, cfg.k, flags)
        guard = 1 << 20
        buf = torch.full((need + 2 * guard,), 0xA5, dtype=torch.uint8, device="cuda")
        ws = buf[guard:guard + need]
        out_buf = torch.full((T + 2, cfg.H), 7.0, dtype=torch.bfloat16, device="cuda")
        ids, tw = moe.route_topk(lg, cfg.k)
        grp = moe.group_tokens(ids, cfg.E)
        moe.mxfp4_ffn(x, w, tw, grp, 0.0, flags, out=out_buf[1:T + 1], workspace=ws)
        torch.cuda.synchronize()
        print(f"guard T={T} flags={flags}", flush=True)
        assert torch.all(buf[:guard] == 0xA5) and torch.all(buf[guard + need:] == 0xA5)
        assert torch.all(out_buf[0] == 7.0) and torch.all(out_buf[T + 1] == 7.0)
