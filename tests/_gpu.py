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
              options=None, ids=None):
    """The whole path on the GPU; returns numpy copies of every intermediate the ABI exposes. With
    `ids` (numpy [T, k]) the router is skipped and those ids are grouped with uniform weights 1/k."""
    x = x_to_device(inp["x"])
    w = w if w is not None else weights_to_device(inp)
    E = w.E
    if ids is None:
        ids, tw = moe.route_topk(dev(inp["logits"]), k, score_fn, renorm)
    else:
        ids = dev(np.asarray(ids, np.int32))
        tw = torch.full(tuple(ids.shape), 1.0 / k, dtype=torch.float32, device="cuda")
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


def assert_output_parity(out_bits_arr, ref, label=""):
    """The output bar, on a bfloat16 output against the unrounded fp64 oracle output `ref`.

    max bar: max|out - ref| <= 2e-2 * rms(ref), asserted literally whenever the exact result
    rounded to bfloat16 meets it (its "floor", max|bf16(ref) - ref| / rms(ref), is below 2e-2).
    Where even the exact result rounded to bfloat16 misses it (heavy-tailed outputs: elements above
    ~8 rms, whose half-ulp exceeds 2e-2 rms), the bar is applied to the error beyond that rounding:
    max_i(|out_i - ref_i| - |bf16(ref_i) - ref_i|) <= 2e-2 * rms(ref).
    mean bar: sum|out - ref| / sum|ref| <= 5e-3, always as printed.
    """
    from _util import bf16_to_f64, parity_metrics, rne_bf16

    m = parity_metrics(out_bits_arr, ref)
    floor = parity_metrics(
        torch.from_numpy(rne_bf16(ref)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16), ref)
    literal = floor["max_raw"] < MAX_ERR_REL_RMS
    msg = (f"{label}: max|err|/rms={m['max_raw']:.3e} (bf16 floor {floor['max_raw']:.3e}), "
           f"excess over own rounding {m['max_excess']:.3e}, "
           f"sum|err|/sum|ref|={m['l1']:.3e} (floor {floor['l1']:.3e}); "
           f"max bar on {'raw error' if literal else 'excess (floor above the bar)'}")
    print(msg, flush=True)
    PARITY_ROWS.append((label, m["max_raw"], floor["max_raw"], m["max_excess"], m["l1"],
                        "raw" if literal else "excess"))
    assert np.all(np.isfinite(bf16_to_f64(out_bits_arr))), msg
    if literal:
        assert m["max_raw"] <= MAX_ERR_REL_RMS, msg
    else:
        assert m["max_excess"] <= MAX_ERR_REL_RMS, msg
    assert m["l1"] <= MEAN_REL_ERR, msg
    return m
