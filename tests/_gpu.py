"""Helpers for the GPU parity tests: run the HIP library through its binding on seeded inputs."""
import math

import numpy as np
import torch

import mxfp4_mixture_experts_amd as moe


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def weights_to_device(inp: dict) -> moe.Mxfp4Weights:
    return moe.Mxfp4Weights(dev(inp["w13_q"]), dev(inp["w13_s"]), dev(inp["w2_q"]), dev(inp["w2_s"]))


def x_to_device(x_bits: np.ndarray) -> torch.Tensor:
    return dev(x_bits.view(np.int16)).view(torch.bfloat16)


def out_bits(out: torch.Tensor) -> np.ndarray:
    return out.view(torch.int16).cpu().numpy().view(np.uint16)


def run_layer(inp: dict, k: int, score_fn: int, clamp: float, flags: int = 0, w=None, renorm=True,
              options=None, ids=None, topk_w=None):
    """The whole path on the GPU; returns numpy copies of every intermediate the ABI exposes. With
    `ids` (numpy [T, k]) the router is skipped and those ids are grouped with the weights `topk_w`
    (numpy [T, k], as float32), uniform 1/k by default."""
    x = x_to_device(inp["x"])
    w = w if w is not None else weights_to_device(inp)
    E = w.E
    if ids is None:
        ids, tw = moe.route_topk(dev(inp["logits"]), k, score_fn, renorm)
    else:
        ids = dev(np.asarray(ids, np.int32))
        if topk_w is None:
            tw = torch.full(tuple(ids.shape), 1.0 / k, dtype=torch.float32, device="cuda")
        else:
            tw = dev(np.asarray(topk_w, np.float32))
    grp = moe.group_tokens(ids, E)
    out = moe.mxfp4_ffn(x, w, tw, grp, clamp, flags, options=options)
    torch.cuda.synchronize()
    T = x.shape[0]
    P = T * k
    n = int(grp.n_active.item())
    return dict(topk_ids=ids.cpu().numpy(), topk_w=tw.cpu().numpy(), counts=grp.counts.cpu().numpy(),
                offsets=grp.offsets.cpu().numpy(), sorted_pair=grp.sorted_pair[:P].cpu().numpy(),
                pair_pos=grp.pair_pos[:P].cpu().numpy(), active_all=grp.active.cpu().numpy(),
                active=grp.active[:n].cpu().numpy(), n_active=n, out_bf16=out_bits(out))


def weight_rtol(n_terms: int) -> float:
    """Relative error bound of a routing weight computed in fp32: exp/sigmoid to ~1 ulp each, a sum of
    n_terms positive terms and one division, each adding at most one rounding of 2^-24 relative."""
    return (n_terms + 4) * 2.0 ** -23


MAX_ERR_REL_RMS = 2e-2   # max |out - ref| <= 2e-2 * rms(ref)
MEAN_REL_ERR = 5e-3      # sum |out - ref| / sum |ref| <= 5e-3

# One row per parity check of this session: label, raw max error, its bf16 floor, the excess over
# the floor, the l1 error and which form of the max bar was asserted. tests/conftest.py prints them
# in the terminal summary.
PARITY_ROWS: list = []


def assert_output_parity(out_bits_arr, ref, label="", allow=None):
    """The output bar, on a bfloat16 output against the unrounded fp64 oracle output `ref`.

    max bar: max|out - ref| <= 2e-2 * rms(ref), asserted literally whenever the exact result
    rounded to bfloat16 meets it (its "floor", max|bf16(ref) - ref| / rms(ref), is below 2e-2).
    Where even the exact result rounded to bfloat16 misses it (heavy-tailed outputs: elements above
    ~8 rms, whose half-ulp exceeds 2e-2 rms), the bar is applied to the error beyond that rounding:
    max_i(|out_i - ref_i| - |bf16(ref_i) - ref_i|) <= 2e-2 * rms(ref).
    mean bar: sum|out - ref| / sum|ref| <= 5e-3, always as printed.
    allow (optional, same shape as ref): a per-element allowance subtracted from |out - ref| before
    the max bar (the outputs that several valid quantisation decisions can reach; see
    mx_flip_allowance); the mean bar takes the raw error.
    """
    from _util import bf16_to_f64, parity_metrics, rne_bf16

    m = parity_metrics(out_bits_arr, ref)
    allow_rms = 0.0
    if allow is not None:
        err = np.abs(bf16_to_f64(out_bits_arr) - ref)
        own = np.abs(rne_bf16(ref) - ref)
        rms = float(np.sqrt(np.mean(ref * ref))) or 1.0
        allow_rms = float(allow.max()) / rms
        m = dict(m, max_raw=float((err - allow).max()) / rms, max_excess=float((err - own - allow).max()) / rms)
    floor = parity_metrics(
        torch.from_numpy(rne_bf16(ref)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16), ref)
    literal = floor["max_raw"] < MAX_ERR_REL_RMS
    msg = (f"{label}: max|err|/rms={m['max_raw']:.3e} (bf16 floor {floor['max_raw']:.3e}), "
           f"excess over own rounding {m['max_excess']:.3e}, "
           f"sum|err|/sum|ref|={m['l1']:.3e} (floor {floor['l1']:.3e}); "
           f"max bar on {'raw error' if literal else 'excess (floor above the bar)'}"
           + (f", beyond a flip allowance of at most {allow_rms:.3e} rms" if allow is not None else ""))
    print(msg, flush=True)
    PARITY_ROWS.append((label, m["max_raw"], floor["max_raw"], m["max_excess"], m["l1"],
                        ("raw" if literal else "excess") + ("-flips" if allow is not None else "")))
    assert np.all(np.isfinite(bf16_to_f64(out_bits_arr))), msg
    if literal:
        assert m["max_raw"] <= MAX_ERR_REL_RMS, msg
    else:
        assert m["max_excess"] <= MAX_ERR_REL_RMS, msg
    assert m["l1"] <= MEAN_REL_ERR, msg
    return m


def sample_tokens(ref_ids, grp, T, k, n=20):
    """Tokens to check at full size: first, last, tokens routed to the most and least loaded active
    experts, and the tokens at the row-tile edges (rows 0, 63, 64, 127, 128, 255, 256, 511, 512,
    767, 768 and the last) of the most loaded expert, so every 64-row MFMA tile boundary and every
    256-row dense tile of it is reached (with one token per row of every expert, as at m1024, of
    every expert); the rest seeded at random."""
    counts, offsets, sorted_pair = grp["counts"], grp["offsets"], grp["sorted_pair"]
    loads = counts[ref_ids].max(axis=1)
    picks = {0, T - 1, int(np.argmax(loads)), int(np.argmin(loads))}
    e = int(np.argmax(counts))
    M = int(counts[e])
    for r in (0, 63, 64, 127, 128, 255, 256, 511, 512, 767, 768, M - 1):
        if 0 <= r < M:
            picks.add(int(sorted_pair[offsets[e] + r]) // k)
    rng = np.random.default_rng(T)
    while len(picks) < n:
        picks.add(int(rng.integers(0, T)))
    return np.array(sorted(picks))


# Relative accumulation error of the block-scaled MFMA, as a fraction of the sum of the absolute
# products: E4M3 operands measured up to 2^-12.6 on codes spanning the whole format (median 2^-14.6);
# E2M1 x E2M1 matched fp32 rounding. The validity check below takes 2^-11 and 2^-20.
MX_ETA = {1: 2.0 ** -11, 2: 2.0 ** -20}


def mx_decode_rows(codes, scales, fmt):
    """Values of quantised rows: codes u8 [n, I] (E4M3) or [n, I/2] (E2M1 pairs), scale bytes [n, I/32]."""
    from _util import E2M1_TABLE

    codes = np.asarray(codes, np.uint8)
    if fmt == 1:
        v = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    else:
        c = np.stack([codes & 0xF, codes >> 4], -1).reshape(codes.shape[0], -1)
        v = np.where(c & 8, -1.0, 1.0) * E2M1_TABLE[c & 7]
    return v * np.repeat(np.exp2(np.asarray(scales, np.float64) - 127.0), 32, axis=1)


def check_mx_h(inp, ids, x_bits, h_pairs, gpu_h, gpu_scales, fmt, clamp):
    """The GPU's quantised h of the pairs of `ids` (rows in pair order) against the oracle's.

    Where they differ, the GPU's decision must be one that its own fp32 h could reach: the gate/up
    sums carry the MFMA's accumulation error (at most eta * sum|x_q| |w|), so h lies in
    [h - dh, h + dh] with dh from the corners of g +- dg, u +- du; the GPU's scale byte must be one that
    the block's maximum over that range gives, and each value must lie between the codes of h - dh and
    h + dh at that scale. Returns (fraction of elements that differ, the GPU's h values)."""
    from _util import bf16_to_f64, dequant, e2m1_bruteforce, e4m3_torch, mx_fake_quant

    eta = MX_ETA[fmt]
    emax = 8 if fmt == 1 else 2
    quant = e4m3_torch if fmt == 1 else e2m1_bruteforce
    xq = mx_fake_quant(bf16_to_f64(x_bits), fmt)
    n, k = ids.shape
    I = inp["w13_q"].shape[1] // 2
    hg = mx_decode_rows(gpu_h, gpu_scales, fmt)
    gs = np.asarray(gpu_scales, np.int64)

    def silu_mul(gg, uu):
        if clamp > 0:
            gg, uu = np.clip(gg, -clamp, clamp), np.clip(uu, -clamp, clamp)
        return gg / (1.0 + np.exp(-gg)) * uu

    def byte_of(amax):
        e = np.floor(np.log2(np.where(amax > 0, amax, 1.0)))
        return np.where(amax > 0, np.clip(e - emax + 127, 0, 254), 0).astype(np.int64)

    differ = 0
    for e in np.unique(ids):
        t_idx, j_idx = np.nonzero(ids == e)
        p = t_idx * k + j_idx
        W13 = dequant(inp["w13_q"][e], inp["w13_s"][e])
        rows = xq[t_idx]
        g, u = rows @ W13[:I].T, rows @ W13[I:].T
        dg = eta * (np.abs(rows) @ np.abs(W13[:I]).T)
        du = eta * (np.abs(rows) @ np.abs(W13[I:]).T)
        h0 = silu_mul(g, u)
        dh = np.zeros_like(h0)
        for sg in (-1.0, 1.0):
            for su in (-1.0, 1.0):
                dh = np.maximum(dh, np.abs(silu_mul(g + sg * dg, u + su * du) - h0))
        h = h_pairs[p]
        dh += np.abs(h0 - h) + 2.0 ** -22 * np.abs(h)
        m = h.shape[0]
        nb = I // 32
        lo = np.nextafter((h - dh).astype(np.float32), np.float32(-np.inf)).astype(np.float64).reshape(m, nb, 32)
        hi = np.nextafter((h + dh).astype(np.float32), np.float32(np.inf)).astype(np.float64).reshape(m, nb, 32)
        hb = h.reshape(m, nb, 32)
        db = dh.reshape(m, nb, 32)
        b_ref = byte_of(np.abs(hb).max(-1))
        b_lo = byte_of(np.maximum(np.abs(hb) - db, 0).max(-1))
        b_hi = byte_of((np.abs(hb) + db).max(-1))
        b_gpu = gs[p].reshape(m, nb)
        bad_scale = (b_gpu < b_lo) | (b_gpu > b_hi)
        assert not bad_scale.any(), f"expert {e}: GPU scale bytes outside the reachable range at {np.argwhere(bad_scale)[:5]}"
        X = np.exp2(b_gpu - 127.0)[..., None]
        vmin = X * quant(lo / X)
        vmax = X * quant(hi / X)
        v = hg[p].reshape(m, nb, 32)
        bad = (v < vmin) | (v > vmax)
        assert not bad.any(), (f"expert {e}: {int(bad.sum())} GPU h codes no fp32 h within the MFMA error "
                               f"reaches, e.g. at {np.argwhere(bad)[:3].tolist()}")
        qref = np.exp2(b_ref - 127.0)[..., None] * quant(hb / np.exp2(b_ref - 127.0)[..., None])
        differ += int(np.count_nonzero(v != qref))
    return differ / float(n * k * I), hg


def mx_conditional_out(inp, ids, wts, hg):
    """The combined output of the down projection on the given h values (rows in pair order), fp64."""
    from _util import dequant

    n, k = ids.shape
    H = inp["w2_q"].shape[1]
    out = np.zeros((n, H))
    for e in np.unique(ids):
        t_idx, j_idx = np.nonzero(ids == e)
        W2 = dequant(inp["w2_q"][e], inp["w2_s"][e])
        np.add.at(out, t_idx, wts[t_idx, j_idx][:, None] * (hg[t_idx * k + j_idx] @ W2.T))
    return out
