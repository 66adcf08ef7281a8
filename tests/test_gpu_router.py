"""GPU parity of the router GEMM + top-k (moe_router_gemm_topk) against the oracle.

The logits are compared with the fp64 oracle logits within the fp32 accumulation bound. The
selection is checked where it is unique whatever the rounding: the ids must equal the oracle's top-k
of the GPU's own logits bit for bit (selection is exact given the logits), the weights must be within
the routing-weight bound, and both must equal moe_route_topk on those logits bitwise (the same device
code). Sizes span ragged token, expert and hidden counts, every expert-count path of the selection
kernel, both GEMM kernels (operands in registers up to 32 tokens, staged through LDS above; K
chunks cut by the slice end), one to sixteen K slices, and the decode and high-concurrency router
shapes."""
import numpy as np
import pytest
import torch

import moe_synth
from _gpu import weight_rtol
from _util import bf16_to_f64

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("mxfp4_mixture_experts_amd")

CASES = [
    # T, H, E, k, score_fn, renorm, seed
    (1, 64, 8, 2, 0, True, 1),
    (8, 4096, 256, 8, 0, True, 2),      # decode M=8 router
    (5, 96, 65, 3, 1, False, 3),
    (70, 544, 130, 6, 0, False, 4),
    (257, 1024, 512, 16, 1, True, 5),
    (33, 7168, 300, 8, 1, True, 6),
    (1024, 7168, 256, 8, 1, True, 7),   # high-concurrency router
    (64, 32, 1, 1, 0, True, 8),         # one K step, one expert
    (24, 2080, 200, 4, 0, True, 11),    # two 16-token blocks per tile
    (32, 160, 64, 2, 1, False, 12),     # the largest batch without LDS staging
]


def bf16_tensor(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "T%d_H%d_E%d_k%d" % c[:4])
def test_router_gemm_topk(orc, case):
    T, H, E, k, fn, renorm, seed = case
    print(f"router gemm T={T} H={H} E={E} k={k} fn={fn} renorm={renorm}", flush=True)
    rng = np.random.Generator(np.random.PCG64(seed))
    x = moe_synth.f32_to_bf16_bits(rng.standard_normal(size=(T, H), dtype=np.float32))
    w = moe_synth.make_router_weights(E, H, seed + 100)
    xg, wg = bf16_tensor(x), bf16_tensor(w)
    ids, tw, logits = moe.router_gemm_topk(xg, wg, k, fn, renorm)
    ids2, tw2, logits2 = moe.router_gemm_topk(xg, wg, k, fn, renorm)
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()

    # logits against fp64: each of the H products is exact in fp32; allow one rounding per product
    # and per slice addition, relative to the sum of the absolute products
    ref = orc.router_logits(x, w)
    mag = np.abs(bf16_to_f64(x)) @ np.abs(bf16_to_f64(w)).T
    bound = (H + 64) * 2.0 ** -24 * mag + 1e-30
    err = np.abs(lg.astype(np.float64) - ref)
    assert np.all(err <= bound), f"max err/bound {np.max(err / bound):.3g}"
    print(f"  max |logit err| {err.max():.3g} (bound {bound.max():.3g})", flush=True)

    # selection: the oracle's top-k of the GPU logits, exactly; weights within the fp32 bound
    oids, ow = orc.route_topk(lg, k, fn, renorm)
    np.testing.assert_array_equal(ids.cpu().numpy(), oids)
    n_terms = k if (renorm or fn == 1) else E
    np.testing.assert_allclose(tw.cpu().numpy(), ow, rtol=weight_rtol(n_terms), atol=0)

    # the same device code as moe_route_topk, and deterministic
    rids, rw = moe.route_topk(logits, k, fn, renorm)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids.cpu().numpy(), rids.cpu().numpy())
    np.testing.assert_array_equal(tw.cpu().numpy().view(np.uint32), rw.cpu().numpy().view(np.uint32))
    np.testing.assert_array_equal(lg.view(np.uint32), logits2.cpu().numpy().view(np.uint32))
    np.testing.assert_array_equal(ids.cpu().numpy(), ids2.cpu().numpy())


def test_router_gemm_without_logits_and_empty():
    rng = np.random.Generator(np.random.PCG64(9))
    T, H, E, k = 8, 256, 32, 4
    x = bf16_tensor(moe_synth.f32_to_bf16_bits(rng.standard_normal(size=(T, H), dtype=np.float32)))
    w = bf16_tensor(moe_synth.make_router_weights(E, H, 10))
    ids_a, w_a, lg = moe.router_gemm_topk(x, w, k)
    ids_b, w_b, none = moe.router_gemm_topk(x, w, k, want_logits=False)
    torch.cuda.synchronize()
    assert none is None
    np.testing.assert_array_equal(ids_a.cpu().numpy(), ids_b.cpu().numpy())
    np.testing.assert_array_equal(w_a.cpu().numpy().view(np.uint32), w_b.cpu().numpy().view(np.uint32))
    ids0, w0, lg0 = moe.router_gemm_topk(x[:0], w, k)
    torch.cuda.synchronize()
    assert ids0.shape == (0, k) and lg0.shape == (0, E)


ONE_LAUNCH = [c for c in CASES if c[0] <= 32]


@pytest.mark.parametrize("case", ONE_LAUNCH, ids=lambda c: "T%d_H%d_E%d_k%d" % c[:4])
def test_one_launch_equals_two_launches(case):
    """Up to 32 tokens the projection and the selection run in one launch: bitwise the logits, ids and
    weights of the two-launch structure, on repeated calls through one workspace (its counter is
    reset by every call) and under HIP-graph replay."""
    T, H, E, k, fn, renorm, seed = case
    rng = np.random.Generator(np.random.PCG64(seed))
    x = bf16_tensor(moe_synth.f32_to_bf16_bits(rng.standard_normal(size=(T, H), dtype=np.float32)))
    w = bf16_tensor(moe_synth.make_router_weights(E, H, seed + 100))
    ws = moe.router_workspace(T, H, E)
    two = moe.router_gemm_topk(x, w, k, fn, renorm, workspace=ws, split_launch=True)
    torch.cuda.synchronize()
    ref = [t.cpu().numpy().view(np.uint32) for t in two]
    for i in range(4):
        print(f"one-launch router T={T} H={H} E={E} k={k} call {i}", flush=True)
        one = moe.router_gemm_topk(x, w, k, fn, renorm, workspace=ws)
        torch.cuda.synchronize()
        for a, b in zip(one, ref):
            np.testing.assert_array_equal(a.cpu().numpy().view(np.uint32), b)
    assert int(ws[:4].cpu().numpy().view(np.uint32)[0]) == 0  # the counter is left at zero
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        gout = moe.router_gemm_topk(x, w, k, fn, renorm, workspace=ws, stream=s)
    for i in range(3):
        for t in gout:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(gout, ref):
            np.testing.assert_array_equal(a.cpu().numpy().view(np.uint32), b)
        moe.router_gemm_topk(x, w, k, fn, renorm, workspace=ws)  # eager call between replays
        torch.cuda.synchronize()
    del ids


LAYER_CASES = [
    # T, H, I, E, k, score_fn, clamp, seed: decode M=8 (one-launch router + grouping), one token,
    # 40 tokens (two router kernels and the grouping kernel), ragged sizes
    (8, 4096, 2048, 256, 8, 0, 0.0, 31),
    (1, 2048, 768, 128, 8, 0, 0.0, 32),
    (40, 512, 256, 16, 4, 1, 7.0, 33),
    (5, 96, 160, 6, 3, 0, 0.0, 34),
]


@pytest.mark.parametrize("case", LAYER_CASES, ids=lambda c: "T%d_H%d_I%d_E%d_k%d" % c[:5])
def test_layer_forward(orc, case):
    """moe_layer_forward (from x and W_router) against the oracle on the GPU's own logits, and bitwise
    against moe_router_gemm_topk + moe_group_tokens + moe_mxfp4_ffn."""
    from _gpu import assert_output_parity, out_bits, weights_to_device, x_to_device

    T, H, I, E, k, fn, clamp, seed = case
    cfg, inp = moe_synth.small_case(T, H, I, E, k, seed, score_fn=fn, clamp=clamp)
    wr_bits = moe_synth.make_router_weights(E, H, seed + 7)
    x = x_to_device(inp["x"])
    wr = bf16_tensor(wr_bits)
    w = weights_to_device(inp)
    ws = moe.layer_forward_workspace(T, H, I, E, k)
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    tw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    print(f"layer_forward T={T} H={H} I={I} E={E} k={k}", flush=True)
    out = moe.layer_forward(x, wr, w, k, fn, True, clamp, workspace=ws, logits=logits, ids=ids, weights=tw)
    out2 = moe.layer_forward(x, wr, w, k, fn, True, clamp, workspace=ws).clone()
    torch.cuda.synchronize()
    # the separate calls
    ids_s, tw_s, lg_s = moe.router_gemm_topk(x, wr, k, fn, True)
    grp = moe.group_tokens(ids_s, E)
    out_s = moe.mxfp4_ffn(x, w, tw_s, grp, clamp)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(logits.cpu().numpy().view(np.uint32), lg_s.cpu().numpy().view(np.uint32))
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_s.cpu().numpy())
    np.testing.assert_array_equal(out_bits(out), out_bits(out_s))
    np.testing.assert_array_equal(out_bits(out2), out_bits(out_s))
    # the oracle on the GPU's logits (selection is exact given the logits)
    ref_logits = orc.router_logits(inp["x"], wr_bits)
    mag = np.abs(bf16_to_f64(inp["x"])) @ np.abs(bf16_to_f64(wr_bits)).T
    assert np.all(np.abs(logits.cpu().numpy().astype(np.float64) - ref_logits) <= (H + 64) * 2.0 ** -24 * mag + 1e-30)
    ref = orc.moe_layer(logits.cpu().numpy(), inp["x"], inp["w13_q"], inp["w13_s"], inp["w2_q"], inp["w2_s"], k, fn,
                        True, clamp)
    np.testing.assert_array_equal(ids.cpu().numpy(), ref["topk_ids"])
    assert_output_parity(out_bits(out), ref["out_ref"], f"layer_forward T{T} H{H} I{I} E{E}")
