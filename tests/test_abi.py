"""The C ABI on the CPU: the library loads, exports every function include/moe_mxfp4.h declares, and
host-side validation returns the documented status codes before anything is launched (no GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mxfp4.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\**\s*(moe_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    import mxfp4_mixture_experts_amd as m

    if not os.path.exists(m.LIB_PATH):
        from mxfp4_mixture_experts_amd import build

        build.build(verbose=False)
    return m.load_library()


# The boundary's entry points as the hot-path scope lists them (route, group with its workspace
# query, the FFN with its workspace query, status strings and the version).
BOUNDARY = ("moe_route_topk", "moe_group_tokens_workspace_size", "moe_group_tokens",
            "moe_mxfp4_ffn_workspace_size", "moe_mxfp4_ffn", "moe_status_string", "moe_abi_version")


def test_header_declares_the_boundary_calls():
    fns = declared_functions()
    for name in BOUNDARY:
        assert name in fns


def test_no_process_wide_setters():
    """Tuning and timing choices are per-call options, not mutable library state."""
    assert not [f for f in declared_functions() if f.startswith("moe_set_")]


def test_every_declared_symbol_is_exported(lib):
    import mxfp4_mixture_experts_amd as m

    out = subprocess.run(["nm", "-D", "--defined-only", m.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (moe_\w+)", out))
    assert set(declared_functions()) == exported


def test_version_and_status_strings(lib):
    assert lib.moe_abi_version() == 2
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.moe_status_string(code)
    assert b"unknown" in lib.moe_status_string(42)


V = ctypes.c_void_p
DUMMY = V(0x1000)  # never dereferenced: every call below fails validation before any launch


def test_route_validation(lib):
    s = None
    assert lib.moe_route_topk(DUMMY, 4, 0, 1, 0, 1, DUMMY, DUMMY, s) == -2  # E < 1
    assert lib.moe_route_topk(DUMMY, 4, 8, 9, 0, 1, DUMMY, DUMMY, s) == -2  # k > E
    assert lib.moe_route_topk(DUMMY, 4, 600, 8, 0, 1, DUMMY, DUMMY, s) == -2  # E > 512
    assert lib.moe_route_topk(DUMMY, 4, 64, 17, 0, 1, DUMMY, DUMMY, s) == -2  # k > 16
    assert lib.moe_route_topk(DUMMY, -1, 8, 2, 0, 1, DUMMY, DUMMY, s) == -2
    assert lib.moe_route_topk(DUMMY, 4, 8, 2, 2, 1, DUMMY, DUMMY, s) == -3  # unknown score fn
    assert lib.moe_route_topk(None, 4, 8, 2, 0, 1, DUMMY, DUMMY, s) == -1
    assert lib.moe_route_topk(DUMMY, 4, 8, 2, 0, 1, None, DUMMY, s) == -1
    assert lib.moe_route_topk(None, 0, 8, 2, 0, 1, None, None, s) == 0  # T == 0: nothing to do


def test_group_validation(lib):
    s = None
    sz = ctypes.c_size_t
    lib.moe_group_tokens_workspace_size.restype = ctypes.c_size_t
    assert lib.moe_group_tokens_workspace_size(8, 8, 256) == 0
    assert lib.moe_group_tokens_workspace_size(0, 8, 256) == 0
    invalid = ctypes.c_size_t(-1).value
    assert lib.moe_group_tokens_workspace_size(4, 2, 0) == invalid
    assert lib.moe_group_tokens_workspace_size(1 << 20, 8, 8) == invalid

    def call(ids=DUMMY, T=4, k=2, E=8, counts=DUMMY, sp=DUMMY, ws=None, ws_bytes=0):
        return lib.moe_group_tokens(ids, T, k, E, counts, DUMMY, sp, DUMMY, DUMMY, DUMMY, ws, sz(ws_bytes), s)

    assert call(E=0) == -2
    assert call(k=0) == -2
    assert call(counts=None) == -1
    assert call(sp=None) == -1
    assert call(ids=None) == -1
    assert call(T=1 << 20, k=8) == -2


def ffn(lib, T=8, H=4096, I=2048, E=256, k=8, x=DUMMY, ws=V(0x10000), ws_bytes=1 << 40, flags=0, out=DUMMY,
        opts=None):
    d = DUMMY
    if opts is None:
        return lib.moe_mxfp4_ffn(x, T, H, I, E, k, d, d, d, d, d, d, d, d, d, d, d, ctypes.c_float(0.0),
                                 flags, out, ws, ws_bytes, None)
    return lib.moe_mxfp4_ffn_ex(x, T, H, I, E, k, d, d, d, d, d, d, d, d, d, d, d, ctypes.c_float(0.0),
                                flags, out, ws, ws_bytes, ctypes.byref(opts), None)


def test_ffn_shape_validation(lib):
    assert ffn(lib, H=4016) == -2  # H % 32
    assert ffn(lib, I=100) == -2
    assert ffn(lib, I=2064) == -2
    assert ffn(lib, H=32768) == -2
    assert ffn(lib, k=9, E=8) == -2
    assert ffn(lib, E=513) == -2
    assert ffn(lib, T=-1) == -2
    assert ffn(lib, T=0, x=None) == 0  # nothing to do


def test_ffn_pointer_alignment_and_flags(lib):
    assert ffn(lib, x=None) == -1
    assert ffn(lib, out=None) == -1
    assert ffn(lib, x=V(0x1008)) == -3  # x not 16-byte aligned
    assert ffn(lib, ws=V(0x10010)) == -3  # workspace not 256-byte aligned
    assert ffn(lib, flags=16) == -3  # unknown flag
    assert ffn(lib, flags=2 | 4) == -3  # both FORCE flags


def test_ffn_workspace_contract(lib):
    lib.moe_mxfp4_ffn_workspace_size.restype = ctypes.c_size_t
    need = lib.moe_mxfp4_ffn_workspace_size(8, 4096, 2048, 256, 8, 0)
    P = 64
    assert need >= P * 2048 * 4 + P * 4096 * 4
    assert ffn(lib, ws_bytes=need - 1) == -4
    unfused = lib.moe_mxfp4_ffn_workspace_size(8, 4096, 2048, 256, 8, 1)
    assert unfused >= need + P * 2048 * 4
    assert lib.moe_mxfp4_ffn_workspace_size(8, 4016, 2048, 256, 8, 0) == 0
    # the size depends only on the sizes and flags, never on a routing: worst case is reserved
    assert lib.moe_mxfp4_ffn_workspace_size(1, 4096, 2048, 256, 8, 0) < need


def test_launch_plan(lib):
    import mxfp4_mixture_experts_amd as m

    p = m.ffn_plan(8, 4096, 2048, 256, 8)
    assert p["launch_small"] == 1 and p["launch_large"] == 0 and p["n_launches"] == 3
    # persistent grid: one workgroup per CU per wave/SIMD (256 CUs when no device can be queried)
    assert p["small_gateup_grid"] % 256 == 0 and p["small_down_grid"] % 256 == 0
    assert m.ffn_plan(1, 2048, 768, 128, 8)["small_gateup_grid"] <= 8 * 768
    p = m.ffn_plan(8, 4096, 2048, 256, 8, m.UNFUSED_GATE_UP)
    assert p["n_launches"] == 4
    assert m.ffn_plan(8, 4096, 2048, 256, 8)["fold_combine"] == 0  # 64 pairs: too many to fold
    # one token, 8 pairs: the combine runs inside the down launch, whose workgroups own whole
    # output-row tiles (7168 rows in tiles of 4)
    p = m.ffn_plan(1, 7168, 2048, 256, 8)
    assert p["fold_combine"] == 1 and p["n_launches"] == 2 and p["combine_grid"] == 0
    assert p["small_down_grid"] == min(7168 // 4, 256)
    p = m.ffn_plan(1, 7168, 2048, 256, 8, m.SEPARATE_COMBINE)
    assert p["fold_combine"] == 0 and p["n_launches"] == 3 and p["combine_grid"] > 0
    assert m.ffn_plan(1, 7168, 2048, 256, 8, m.UNFUSED_GATE_UP)["n_launches"] == 3
    assert m.ffn_plan(1, 7168, 2048, 256, 8, m.FORCE_LARGE_M)["fold_combine"] == 0
    p = m.ffn_plan(1024, 7168, 2048, 256, 8)
    # from 256 tokens every expert runs on the MFMA kernels: schedule, row-tile gate_up + down, dense
    # gate_up + h rewrite + down, combine
    assert p["small_m_max"] == 0 and p["launch_small"] == 0 and p["launch_large"] == 1 and p["n_launches"] == 7
    p = m.ffn_plan(255, 7168, 2048, 256, 8)
    # streaming gate_up + down as well, and no dense kernels below 256 tokens
    assert p["small_m_max"] == 2 and p["launch_small"] == 1 and p["launch_large"] == 1 and p["n_launches"] == 6
    p = m.ffn_plan(64, 4096, 2048, 256, 8, options=m.ffn_options(small_m_max=0))
    assert p["launch_small"] == 0 and p["launch_large"] == 1
    p = m.ffn_plan(1024, 7168, 2048, 256, 8, m.FORCE_LARGE_M)
    assert p["launch_small"] == 0 and p["launch_large"] == 1 and p["small_m_max"] == 0
    p = m.ffn_plan(1024, 7168, 2048, 256, 8, m.FORCE_SMALL_M)
    assert p["launch_large"] == 0
    p = m.ffn_plan(0, 4096, 2048, 256, 8)
    assert p["n_launches"] == 0
    assert m.ffn_plan(8, 4096, 2048, 256, 8)["small_m_max"] == 8
    assert m.ffn_plan(9, 4096, 2048, 256, 8)["small_m_max"] == 2
    assert m.ffn_plan(256, 4096, 2048, 256, 8)["small_m_max"] == 0
    assert m.ffn_plan(8, 4096, 2048, 256, 8, options=m.ffn_options(small_m_max=2))["launch_large"] == 1
    assert m.ffn_plan(8, 4096, 2048, 256, 8)["launch_large"] == 0  # nothing persists between calls
    with pytest.raises(m.MoeError):
        m.ffn_plan(8, 4096, 2048, 256, 8, 6)
    with pytest.raises(m.MoeError):
        m.ffn_plan(8, 4096, 2048, 256, 8, options=m.ffn_options(small_m_max=-2))


def test_ffn_options_validation(lib):
    import mxfp4_mixture_experts_amd as m

    o = m.FfnOptions()
    lib.moe_ffn_options_init(ctypes.byref(o))
    assert o.small_m_max == -1 and o.dense_down_cols == 0
    assert all(v is None for v in o.stage_start) and all(v is None for v in o.stage_stop)
    for bad in (-1, 1, 128, 255, 512):
        assert ffn(lib, opts=m.ffn_options(dense_down_cols=bad)) == -2
    assert ffn(lib, opts=m.ffn_options(small_m_max=-5)) == -2
    # valid options pass validation (the call then fails on its NULL output only)
    assert ffn(lib, out=None, opts=m.ffn_options(dense_down_cols=224, small_m_max=0)) == -1


def test_router_gemm_validation(lib):
    lib.moe_router_gemm_topk_workspace_size.restype = ctypes.c_size_t
    assert lib.moe_router_gemm_topk_workspace_size(8, 4096, 256) >= 8 * 256 * 4
    assert lib.moe_router_gemm_topk_workspace_size(8, 4016, 256) == 0  # H % 32
    assert lib.moe_router_gemm_topk_workspace_size(8, 4096, 513) == 0  # E > MOE_MAX_EXPERTS
    need = lib.moe_router_gemm_topk_workspace_size(8, 4096, 256)
    sz = ctypes.c_size_t
    call = lambda **kw: lib.moe_router_gemm_topk(  # noqa: E731
        kw.get("x", DUMMY), kw.get("w", DUMMY), kw.get("T", 8), kw.get("H", 4096), kw.get("E", 256),
        kw.get("k", 8), kw.get("fn", 0), 1, None, kw.get("ids", DUMMY), DUMMY, kw.get("ws", DUMMY),
        sz(kw.get("ws_bytes", need)), None)
    assert call(H=96 + 16) == -2            # H % 32
    assert call(k=9, E=8) == -2             # k > E
    assert call(fn=3) == -3                 # unknown score function
    assert call(T=0) == 0                   # nothing to do, nothing launched
    assert call(x=None) == -1
    assert call(ids=None) == -1
    assert call(x=V(0x1008)) == -3          # x not 16-byte aligned
    assert call(ws=V(0x1010)) == -3         # workspace not 256-byte aligned
    assert call(ws_bytes=need - 1) == -4


def test_noalloc_validation(lib):
    """The no-allocation entry point rejects bad sizes, and shapes whose workspace exceeds its fixed
    scratch, before touching the GPU."""
    lib.moe_mxfp4_ffn_noalloc_max_bytes.restype = ctypes.c_size_t
    lib.moe_mxfp4_ffn_workspace_size.restype = ctypes.c_size_t
    cap = lib.moe_mxfp4_ffn_noalloc_max_bytes()
    assert cap == 16 << 20
    assert lib.moe_mxfp4_ffn_workspace_size(85, 4096, 2048, 256, 8, 0) <= cap
    assert lib.moe_mxfp4_ffn_workspace_size(86, 4096, 2048, 256, 8, 0) > cap
    d = DUMMY

    def call(T=8, H=4096, I=2048, E=256, k=8, flags=0):
        return lib.moe_mxfp4_ffn_noalloc(d, T, H, I, E, k, d, d, d, d, d, d, d, d, d, d, d, ctypes.c_float(0.0),
                                         flags, d, None)

    assert call(T=86) == -4           # workspace beyond the scratch
    assert call(T=1024, H=7168) == -4
    assert call(H=4016) == -2
    assert call(flags=16) == -3
    assert call(T=0) == 0             # nothing to do


def test_layer_from_logits_validation(lib):
    """moe_layer_from_logits: sizes, flags, pointers and workspace are checked before any launch; the
    routed query follows the gate_up variant's limits."""
    lib.moe_layer_from_logits_workspace_size.restype = ctypes.c_size_t
    lib.moe_mxfp4_ffn_workspace_size.restype = ctypes.c_size_t
    need = lib.moe_layer_from_logits_workspace_size(8, 4096, 2048, 256, 8, 0)
    # routing and grouping arrays (P ids, P weights, E counts, E + 1 offsets, P sorted pairs, P positions,
    # E active, 1 count, each 256-byte aligned), then the FFN's workspace
    assert need > lib.moe_mxfp4_ffn_workspace_size(8, 4096, 2048, 256, 8, 0)
    assert lib.moe_layer_from_logits_workspace_size(8, 4016, 2048, 256, 8, 0) == 0   # H % 32
    assert lib.moe_layer_from_logits_workspace_size(8, 4096, 2048, 256, 8, 16) == 0  # unknown flag
    # one token, 8 pairs, 128 experts, x in 4 KB: routed inside gate_up (also with no device to ask)
    assert lib.moe_layer_from_logits_routed(1, 2048, 768, 128, 8, 0, None) == 1
    assert lib.moe_layer_from_logits_routed(1, 2048, 768, 128, 8, 1, None) == 0     # unfused gate/up
    assert lib.moe_layer_from_logits_routed(1, 2048, 768, 128, 8, 4, None) == 0     # MFMA kernels
    assert lib.moe_layer_from_logits_routed(16, 2048, 768, 128, 8, 0, None) == 0    # 128 pairs
    assert lib.moe_layer_from_logits_routed(1, 2048, 768, 512, 8, 0, None) == 0     # more than 256 experts
    assert lib.moe_layer_from_logits_routed(0, 2048, 768, 128, 8, 0, None) == 0
    from mxfp4_mixture_experts_amd import FfnOptions

    opts = FfnOptions()
    lib.moe_ffn_options_init(ctypes.byref(opts))
    opts.small_m_max = 0                                                          # MFMA kernels
    assert lib.moe_layer_from_logits_routed(1, 2048, 768, 128, 8, 0, ctypes.byref(opts)) == 0
    opts.small_m_max = -2                                                         # invalid options
    assert lib.moe_layer_from_logits_routed(1, 2048, 768, 128, 8, 0, ctypes.byref(opts)) == 0
    d = DUMMY
    sz = ctypes.c_size_t

    def call(T=8, H=4096, I=2048, E=256, k=8, fn=0, flags=0, logits=d, out=d, ws=V(0x10000), ws_bytes=need,
             o=None):
        return lib.moe_layer_from_logits(logits, d, T, H, I, E, k, fn, 1, d, d, d, d, ctypes.c_float(0.0), flags,
                                         None, None, out, ws, sz(ws_bytes), o, None)

    assert call(H=4016) == -2
    assert call(k=9, E=8) == -2
    assert call(fn=2) == -3
    assert call(flags=16) == -3
    assert call(flags=2 | 4) == -3
    assert call(logits=None) == -1
    assert call(out=None) == -1
    assert call(ws=V(0x10010)) == -3
    assert call(ws_bytes=need - 1) == -4
    assert call(o=ctypes.byref(opts)) == -2                                       # small_m_max -2
    assert call(T=0) == 0


def test_layer_decode_validation(lib):
    """moe_layer_decode: sizes, support limits, pointers and workspace are checked before any launch."""
    lib.moe_layer_decode_workspace_size.restype = ctypes.c_size_t
    need = lib.moe_layer_decode_workspace_size(8, 4096, 2048, 256, 8)
    # 256 bytes of barrier state, then (T * CUs + 2 T k) rows of H fp32 partial outputs (256 CUs here)
    assert need == 256 + (8 * 256 + 2 * 64) * 4096 * 4
    assert lib.moe_layer_decode_workspace_size(17, 4096, 2048, 256, 8) == 0   # T > 16
    assert lib.moe_layer_decode_workspace_size(16, 4096, 2048, 256, 16) == 0  # share > 32 blocks
    assert lib.moe_layer_decode_workspace_size(8, 4016, 2048, 256, 8) == 0    # H % 32
    d = DUMMY
    sz = ctypes.c_size_t

    def call(T=8, H=4096, I=2048, E=256, k=8, fn=0, logits=d, out=d, ws=V(0x10000), ws_bytes=need):
        return lib.moe_layer_decode(logits, d, T, H, I, E, k, fn, 1, d, d, d, d, ctypes.c_float(0.0), None, None,
                                    out, ws, sz(ws_bytes), None)

    assert call(H=4016) == -2
    assert call(k=9, E=8) == -2
    assert call(fn=2) == -3
    assert call(T=17) == -3
    assert call(logits=None) == -1
    assert call(out=None) == -1
    assert call(ws=V(0x10010)) == -3
    assert call(ws_bytes=need - 1) == -4
    assert call(T=0) == 0


def test_router_and_layer_forward_validation(lib):
    lib.moe_router_gemm_topk_workspace_size.restype = ctypes.c_size_t
    lib.moe_layer_forward_workspace_size.restype = ctypes.c_size_t
    # a 256-byte header (the one-launch router's counter) before the partial logits
    assert lib.moe_router_gemm_topk_workspace_size(8, 4096, 256) >= 256 + 8 * 256 * 4
    need = lib.moe_layer_forward_workspace_size(8, 4096, 2048, 256, 8, 0)
    assert need > lib.moe_mxfp4_ffn_workspace_size(8, 4096, 2048, 256, 8, 0)
    assert lib.moe_layer_forward_workspace_size(8, 4016, 2048, 256, 8, 0) == 0
    d = DUMMY
    sz = ctypes.c_size_t
    assert lib.moe_router_gemm_topk_ex(d, d, 8, 4096, 256, 8, 0, 1, None, d, d, d, sz(1 << 30), 2, None) == -3

    def call(T=8, H=4096, I=2048, E=256, k=8, fn=0, flags=0, out=d, ws=V(0x10000), ws_bytes=need):
        return lib.moe_layer_forward(d, d, T, H, I, E, k, fn, 1, d, d, d, d, ctypes.c_float(0.0), flags, None, None,
                                     None, out, ws, sz(ws_bytes), None)

    assert call(H=4016) == -2
    assert call(fn=2) == -3
    assert call(flags=6) == -3
    assert call(out=None) == -1
    assert call(ws=V(0x10010)) == -3
    assert call(ws_bytes=need - 1) == -4
    assert call(T=0) == 0


def test_mx_quantize_validation(lib):
    s = None
    assert lib.moe_mx_quantize(DUMMY, -1, 64, 1, DUMMY, DUMMY, s) == -2
    assert lib.moe_mx_quantize(DUMMY, 4, 48, 1, DUMMY, DUMMY, s) == -2   # cols % 32
    assert lib.moe_mx_quantize(DUMMY, 4, 0, 1, DUMMY, DUMMY, s) == -2
    assert lib.moe_mx_quantize(DUMMY, 4, 64, 3, DUMMY, DUMMY, s) == -3   # unknown format
    assert lib.moe_mx_quantize(DUMMY, 4, 64, 0, DUMMY, DUMMY, s) == -3
    assert lib.moe_mx_quantize(None, 0, 64, 2, None, None, s) == 0       # nothing to do
    assert lib.moe_mx_quantize(None, 4, 64, 1, DUMMY, DUMMY, s) == -1
    assert lib.moe_mx_quantize(DUMMY, 4, 64, 1, DUMMY, None, s) == -1
    assert lib.moe_mx_quantize(V(0x1008), 4, 64, 1, DUMMY, DUMMY, s) == -3  # x not 16-byte aligned
    assert lib.moe_mx_quantize(DUMMY, 4, 64, 2, V(0x1004), DUMMY, s) == -3  # codes not 16-byte aligned


def test_ffn_mx_workspace_and_validation(lib):
    q = lib.moe_mxfp4_ffn_mx_workspace_size
    assert q(8, 96, 128, 4, 2, 1) == 0      # H % 128
    assert q(8, 128, 160, 4, 2, 1) == 0     # I % 128
    assert q(8, 128, 128, 4, 2, 0) == 0     # format
    assert q(8, 128, 128, 4, 5, 1) == 0     # k > E
    w8, w4 = q(1024, 7168, 2048, 8, 8, 1), q(1024, 7168, 2048, 8, 8, 2)
    assert w8 > w4 > 1024 * 8 * 7168 * 4   # y alone is P*H fp32
    s = None

    def call(T=8, H=256, I=256, E=4, k=2, act=1, x=DUMMY, w13s=DUMMY, ws=DUMMY, wsb=1 << 30, out=DUMMY):
        return lib.moe_mxfp4_ffn_mx(x, T, H, I, E, k, DUMMY, w13s, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY,
                                    DUMMY, ctypes.c_float(0.0), act, out, ws, wsb, None, s)
    assert call(H=96) == -2
    assert call(I=160) == -2
    assert call(k=5) == -2
    assert call(act=0) == -3
    assert call(act=3) == -3
    assert call(T=0, x=None, out=None, ws=None) == 0
    assert call(x=None) == -1
    assert call(ws=None) == -1
    assert call(w13s=V(0x1002)) == -3       # scales not 4-byte aligned
    assert call(ws=V(0x1080)) == -3         # workspace not 256-byte aligned
    assert call(wsb=q(8, 256, 256, 4, 2, 1) - 1) == -4
