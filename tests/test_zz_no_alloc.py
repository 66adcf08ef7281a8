"""moe_mxfp4_ffn_noalloc (the entry point that allocates nothing: its workspace is the library's
file-scope device scratch) against moe_mxfp4_ffn with a caller's workspace: bitwise equal, and
within the output bar of the oracle, on two calls in a row, the second with a smaller input (the
scratch keeps the first call's contents, which the second must not depend on)."""
import ctypes

import numpy as np
import pytest
import torch

import moe_synth
from _gpu import assert_output_parity, dev, out_bits, weights_to_device, x_to_device

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("mxfp4_mixture_experts_amd")


def noalloc_call(lib, x, w, tw, grp, clamp, flags, out):
    """One moe_mxfp4_ffn_noalloc call straight through the C ABI (ctypes)."""
    T, H = x.shape
    k = tw.shape[1]
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    return lib.moe_mxfp4_ffn_noalloc(
        p(x), T, H, w.I, w.E, k, p(w.w13_q), p(w.w13_s), p(w.w2_q), p(w.w2_s), p(tw), p(grp.counts),
        p(grp.offsets), p(grp.sorted_pair), p(grp.pair_pos), p(grp.active), p(grp.n_active),
        ctypes.c_float(clamp), flags, p(out), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


# (T, H, I, E, k, seed, clamp, flags) of the first call, then of the second (smaller) call
SEQUENCES = [
    ((8, 4096, 2048, 64, 8, 61, 0.0, 0), (2, 4096, 2048, 64, 8, 62, 0.0, 0)),
    ((40, 1024, 512, 8, 4, 63, 7.0, 0), (5, 512, 256, 8, 2, 64, 0.0, moe.UNFUSED_GATE_UP)),
    ((300, 256, 128, 2, 2, 65, 0.0, 0), (17, 256, 128, 4, 2, 66, 0.0, moe.FORCE_LARGE_M)),
]


@pytest.mark.parametrize("seq", SEQUENCES, ids=lambda s: "T%d_then_T%d" % (s[0][0], s[1][0]))
def test_noalloc_matches_workspace_call(orc, seq):
    lib = moe.load_library()
    assert lib.moe_mxfp4_ffn_noalloc_max_bytes() == 16 << 20
    for T, H, I, E, k, seed, clamp, flags in seq:
        cfg, inp = moe_synth.small_case(T, H, I, E, k, seed, clamp=clamp)
        assert moe.ffn_workspace_size(T, H, I, E, k, flags) <= lib.moe_mxfp4_ffn_noalloc_max_bytes()
        w = weights_to_device(inp)
        x = x_to_device(inp["x"])
        ids, tw = moe.route_topk(dev(inp["logits"]), k)
        grp = moe.group_tokens(ids, E)
        ref_out = moe.mxfp4_ffn(x, w, tw, grp, clamp, flags)
        out = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device="cuda")
        print(f"noalloc T={T} H={H} I={I} E={E} k={k} flags={flags}", flush=True)
        assert noalloc_call(lib, x, w, tw, grp, clamp, flags, out) == 0
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out_bits(out), out_bits(ref_out))
        ref = orc.moe_layer(inp["logits"], inp["x"], inp["w13_q"], inp["w13_s"], inp["w2_q"], inp["w2_s"],
                            k, 0, True, clamp)
        assert_output_parity(out_bits(out), ref["out_ref"], f"noalloc T{T} H{H} I{I} flags={flags}")


def test_noalloc_rejects_shapes_beyond_the_scratch():
    lib = moe.load_library()
    d = ctypes.c_void_p(0x1000)  # never dereferenced: the size check fails before any launch
    # T = 1024 at H = 7168, I = 2048 needs about 290 MB of workspace
    rc = lib.moe_mxfp4_ffn_noalloc(d, 1024, 7168, 2048, 256, 8, d, d, d, d, d, d, d, d, d, d, d,
                                   ctypes.c_float(0.0), 0, d, None)
    assert rc == -4
