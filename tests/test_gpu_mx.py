"""GPU parity of the activation-quantised path (moe_mx_quantize, moe_mxfp4_ffn_mx) against the oracle's
activation-quantised mode.

* moe_mx_quantize: codes and scale bytes bit for bit against the oracle's block quantiser (both take
  every decision from the exact bfloat16 value), on normal rows, rows whose blocks span 2^+-60, and
  hand-built blocks (zeros, ties of both formats, saturation, bfloat16 extremes and subnormals);
* moe_mxfp4_ffn_mx, W4A8 and W4A4, on ragged shapes (several 256-row tiles and partial ones, partial
  down column tiles, empty experts, clamp, sigmoid routing) and at the full per-expert M = 1024
  workload on sampled tokens, deterministic across calls. The GPU decides h's codes from its own fp32
  h, the oracle from its fp64 h rounded to binary32; where h lies within the GEMM's accumulation error
  of a rounding boundary both decisions are correct. So the check is in three parts: every GPU h code
  equals the oracle's or is one that an fp32 h within that error reaches (and few differ); the output
  meets the bar against the oracle's down projection and combine on the GPU's own h; and it meets the
  bar against the oracle's output beyond the difference those valid decisions make.
"""
import numpy as np
import pytest
import torch

import moe_synth
from _gpu import (assert_output_parity, check_mx_h, dev, mx_conditional_out, out_bits, sample_tokens,
                  weights_to_device, x_to_device)

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("mxfp4_mixture_experts_amd")

FMTS = {"w4a8": 1, "w4a4": 2}


def bf16_bits(a):
    return moe_synth.f32_to_bf16_bits(np.asarray(a, np.float32))


def oracle_quant(orc, x_bits, fmt):
    """The oracle's codes (packed as the library packs them) and scale bytes of every 32-block."""
    from _util import bf16_to_f64

    v = bf16_to_f64(x_bits)
    R, C = v.shape
    codes = np.zeros((R, C if fmt == 1 else C // 2), np.uint8)
    scales = np.zeros((R, C // 32), np.uint8)
    for r in range(R):
        for b in range(C // 32):
            s, c = orc.mx_quantize_block(v[r, 32 * b:32 * b + 32], fmt)
            scales[r, b] = s
            if fmt == 1:
                codes[r, 32 * b:32 * b + 32] = c
            else:
                codes[r, 16 * b:16 * b + 16] = c[0::2] | (c[1::2] << 4)
    return codes, scales


def special_blocks():
    rows = []
    z = np.zeros(32)
    rows.append(z.copy())                                   # zero block
    b = z.copy(); b[5] = -3.0; rows.append(b)               # one value
    b = z.copy(); b[:10] = [256, 9.0, 8.5, 9.5, 2 ** -10, 3 * 2 ** -10, 2 ** -6, 7 * 2 ** -9, -5.5, 0.1]
    rows.append(b)                                          # E4M3 ties and subnormals at scale 2^0
    b = z.copy(); b[:9] = [5.0, 0.3, 2.5, -0.75, 1.25, -1.75, 3.5, 0.25, -0.2]; rows.append(b)  # E2M1 ties
    b = z.copy(); b[:4] = [500, 480, 449, -300]; rows.append(b)                  # E4M3 saturation
    b = z.copy(); b[:3] = [7.0, 6.5, -7.0]; rows.append(b)                        # E2M1 saturation
    b = z.copy(); b[:2] = [3.3895314e38, -1.0e38]; rows.append(b)                # bf16 largest
    b = z.copy(); b[:3] = [2.0 ** -133, 2.0 ** -126, -2.0 ** -130]; rows.append(b)  # bf16 subnormals
    b = np.full(32, -0.0); b[0] = 1e-3; rows.append(b)      # signed zeros
    return np.array(rows)


@pytest.mark.parametrize("fmt_name", list(FMTS))
def test_mx_quantize_bitwise(orc, fmt_name):
    fmt = FMTS[fmt_name]
    rng = np.random.default_rng(40 + fmt)
    normal = rng.standard_normal((37, 256))
    wide = rng.standard_normal((11, 512)) * np.repeat(np.exp2(rng.uniform(-60, 60, (11, 16))), 32, axis=1)
    special = np.concatenate([special_blocks(), np.zeros((1, 32))]).reshape(-1, 64)
    for name, arr in (("normal", normal), ("wide", wide), ("special", special)):
        xb = bf16_bits(arr)
        print(f"mx_quantize {fmt_name} {name} {xb.shape}", flush=True)
        codes, scales = moe.mx_quantize(x_to_device(xb), fmt)
        torch.cuda.synchronize()
        oc, osc = oracle_quant(orc, xb, fmt)
        np.testing.assert_array_equal(scales.cpu().numpy(), osc)
        np.testing.assert_array_equal(codes.cpu().numpy(), oc)


MX_CASES = [
    # T, H, I, E, k, score_fn, clamp, seed
    (64, 256, 256, 4, 2, 0, 0.0, 1),      # ~32 rows per expert: one partial tile each
    (300, 512, 384, 3, 2, 0, 0.0, 2),     # ~200 rows per expert, three gate_up column tiles
    (7, 128, 128, 5, 3, 1, 0.0, 3),       # tiny; H = 128: half of the one down column tile
    (600, 384, 256, 2, 1, 0, 4.0, 4),     # ~300 rows per expert: a full and a partial tile; clamp;
                                          # H = 384: a full and a half down column tile
    (40, 1024, 512, 16, 4, 0, 0.0, 5),    # 16 experts, some empty
    (520, 256, 128, 1, 1, 0, 0.0, 6),     # one expert, 520 rows: three tiles
]


def run_mx(inp, k, score_fn, clamp, fmt, w=None, repeat=1):
    """The GPU path; returns ids, the outputs of `repeat` calls, and the quantised h of the last call
    (codes and scale bytes, rows in pair order)."""
    x = x_to_device(inp["x"])
    w = w if w is not None else weights_to_device(inp)
    ids, tw = moe.route_topk(dev(inp["logits"]), k, score_fn, True)
    grp = moe.group_tokens(ids, w.E)
    T, H = x.shape
    ws = torch.empty(moe.ffn_mx_workspace_size(T, H, w.I, w.E, k, fmt), dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(repeat):
        outs.append(out_bits(moe.mxfp4_ffn_mx(x, w, tw, grp, clamp, fmt, workspace=ws)))
    codes, scales = moe.ffn_mx_h_view(ws, T, H, w.I, w.E, k, fmt)
    pos = grp.pair_pos[:T * k].long()
    hc, hs = codes[pos].cpu().numpy(), scales[pos].cpu().numpy()
    torch.cuda.synchronize()
    return ids.cpu().numpy(), outs, hc, hs


def check_mx_outputs(inp, oids, ow, x_bits, out, hc, hs, fmt, clamp, label, max_differ):
    """h decisions valid, down + combine exact given the GPU's h, and the output against the oracle
    beyond what the GPU's own (valid) h decisions explain."""
    ref = orc_ffn(inp, oids, ow, x_bits, fmt, clamp)
    frac, hg = check_mx_h(inp, oids, x_bits, ref["h_pairs"], hc, hs, fmt, clamp)
    print(f"{label}: {frac:.2e} of h elements decided differently (each within the MFMA error of a "
          f"boundary)", flush=True)
    assert frac <= max_differ
    cond = mx_conditional_out(inp, oids, ow, hg)
    assert_output_parity(out, cond, f"{label} | GPU h")
    assert_output_parity(out, ref["out_ref"], label, allow=np.abs(cond - ref["out_ref"]))


def orc_ffn(inp, ids, wts, x_bits, fmt, clamp):
    import oracle

    return oracle.default().mxfp4_ffn(x_bits, inp["w13_q"], inp["w13_s"], inp["w2_q"], inp["w2_s"], ids, wts, clamp,
                                      act_fmt=fmt, want_h=True)


MAX_DIFFER = {1: 1e-2, 2: 1e-3}


@pytest.mark.parametrize("fmt_name", list(FMTS))
@pytest.mark.parametrize("case", MX_CASES, ids=lambda c: "T%d_H%d_I%d_E%d_k%d" % c[:5])
def test_ffn_mx_parity(orc, case, fmt_name):
    T, H, I, E, k, fn, clamp, seed = case
    fmt = FMTS[fmt_name]
    cfg, inp = moe_synth.small_case(T, H, I, E, k, seed, score_fn=fn, clamp=clamp)
    print(f"ffn_mx {fmt_name} T={T} H={H} I={I} E={E} k={k} clamp={clamp}", flush=True)
    ids, (o1, o2), hc, hs = run_mx(inp, k, fn, clamp, fmt, repeat=2)
    oids, ow = orc.route_topk(inp["logits"], k, fn)
    np.testing.assert_array_equal(ids, oids)
    np.testing.assert_array_equal(o1, o2)  # deterministic
    check_mx_outputs(inp, oids, ow, inp["x"], o1, hc, hs, fmt, clamp, f"mx {fmt_name} T{T} H{H} I{I} E{E} k{k}",
                     MAX_DIFFER[fmt])


@pytest.mark.parametrize("fmt_name", list(FMTS))
def test_ffn_mx_m1024_sampled(orc, fmt_name):
    fmt = FMTS[fmt_name]
    cfg = moe_synth.CONFIGS["m1024"]
    inp = moe_synth.make_inputs(cfg)
    ids, wts = orc.route_topk(inp["logits"], cfg.k, cfg.score_fn, cfg.renorm)
    grp = orc.group_tokens(ids, cfg.E)
    toks = sample_tokens(ids, grp, cfg.T, cfg.k, n=12)
    print(f"ffn_mx {fmt_name} m1024 sampled tokens {toks.tolist()}", flush=True)
    gids, (out,), hc, hs = run_mx(inp, cfg.k, cfg.score_fn, cfg.clamp, fmt)
    np.testing.assert_array_equal(gids, ids)
    rows = (toks[:, None] * cfg.k + np.arange(cfg.k)).reshape(-1)
    check_mx_outputs(inp, ids[toks], wts[toks], inp["x"][toks], out[toks], hc[rows], hs[rows], fmt, cfg.clamp,
                     f"mx {fmt_name} m1024 ({len(toks)} tokens)", MAX_DIFFER[fmt])


def test_ffn_mx_empty_batch():
    cfg, inp = moe_synth.small_case(4, 128, 128, 2, 1, 9)
    w = weights_to_device(inp)
    x = x_to_device(inp["x"])[:0]
    ids = torch.zeros((0, 1), dtype=torch.int32, device="cuda")
    tw = torch.zeros((0, 1), dtype=torch.float32, device="cuda")
    grp = moe.group_tokens(ids, 2)
    out = moe.mxfp4_ffn_mx(x, w, tw, grp, 0.0, 1)
    torch.cuda.synchronize()
    assert out.shape == (0, 128)
