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


def run_layer(inp: dict, k: int, score_fn: int, clamp: float, flags: int = 0, w=None, renorm=True):
    """The whole path on the GPU; returns numpy copies of every intermediate the ABI exposes."""
    logits = dev(inp["logits"])
    x = x_to_device(inp["x"])
    w = w if w is not None else weights_to_device(inp)
    E = w.E
    ids, tw = moe.route_topk(logits, k, score_fn, renorm)
    grp = moe.group_tokens(ids, E)
    out = moe.mxfp4_ffn(x, w, tw, grp, clamp, flags)
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


MAX_ERR_REL_RMS = 2e-2   # max |out - ref| beyond bf16(ref)'s own rounding <= 2e-2 * rms(ref)
MEAN_REL_ERR = 5e-3      # sum |out - ref| / sum |ref| <= 5e-3


def assert_output_parity(out_bits_arr, ref, label=""):
    from _util import bf16_to_f64, parity_metrics, rne_bf16

    m = parity_metrics(out_bits_arr, ref)
    floor = parity_metrics(
        torch.from_numpy(rne_bf16(ref)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16), ref)
    msg = (f"{label}: max|err|/rms={m['max_raw']:.3e} (bf16 floor {floor['max_raw']:.3e}), "
           f"excess over own rounding {m['max_excess']:.3e}, "
           f"sum|err|/sum|ref|={m['l1']:.3e} (floor {floor['l1']:.3e})")
    print(msg, flush=True)
    assert np.all(np.isfinite(bf16_to_f64(out_bits_arr))), msg
    assert m["max_excess"] <= MAX_ERR_REL_RMS, msg
    assert m["l1"] <= MEAN_REL_ERR, msg
    return m
