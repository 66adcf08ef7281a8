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


def test_header_declares_the_three_calls():
    fns = declared_functions()
    for name in ("moe_route_topk", "moe_group_tokens", "moe_mxfp4_ffn", "moe_mxfp4_ffn_workspace_size"):
        assert name in fns


def test_every_declared_symbol_is_exported(lib):
    import mxfp4_mixture_experts_amd as m

    out = subprocess.run(["nm", "-D", "--defined-only", m.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (moe_\w+)", out))
    assert set(declared_functions()) == exported


def test_version_and_status_strings(lib):
    assert lib.moe_abi_version() == 1
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
    assert lib.moe_group_tokens(DUMMY, 4, 2, 0, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, s) == -2
    assert lib.moe_group_tokens(DUMMY, 4, 0, 8, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, s) == -2
    assert lib.moe_group_tokens(DUMMY, 4, 2, 8, None, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, s) == -1
    assert lib.moe_group_tokens(DUMMY, 4, 2, 8, DUMMY, DUMMY, None, DUMMY, DUMMY, DUMMY, s) == -1
    assert lib.moe_group_tokens(None, 4, 2, 8, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, s) == -1
    assert lib.moe_group_tokens(DUMMY, 1 << 20, 8, 8, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, s) == -2


def ffn(lib, T=8, H=4096, I=2048, E=256, k=8, x=DUMMY, ws=V(0x10000), ws_bytes=1 << 40, flags=0, out=DUMMY):
    d = DUMMY
    return lib.moe_mxfp4_ffn(x, T, H, I, E, k, d, d, d, d, d, d, d, d, d, d, d, ctypes.c_float(0.0),
                             flags, out, ws, ws_bytes, None)


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
    assert ffn(lib, flags=8) == -3  # unknown flag
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
    p = m.ffn_plan(1024, 7168, 2048, 256, 8)
    # schedule, streaming gate_up + down, row-tile gate_up + down, dense gate_up + h rewrite + down,
    # combine
    assert p["launch_small"] == 1 and p["launch_large"] == 1 and p["n_launches"] == 9
    p = m.ffn_plan(1024, 7168, 2048, 256, 8, m.FORCE_LARGE_M)
    assert p["launch_small"] == 0 and p["launch_large"] == 1 and p["small_m_max"] == 0
    p = m.ffn_plan(1024, 7168, 2048, 256, 8, m.FORCE_SMALL_M)
    assert p["launch_large"] == 0
    p = m.ffn_plan(0, 4096, 2048, 256, 8)
    assert p["n_launches"] == 0
    assert m.ffn_plan(8, 4096, 2048, 256, 8)["small_m_max"] == 8
    assert m.ffn_plan(256, 4096, 2048, 256, 8)["small_m_max"] == 2
    prev = m.set_small_m_max(2)
    try:
        assert prev == -1
        assert m.ffn_plan(8, 4096, 2048, 256, 8)["launch_large"] == 1
    finally:
        m.set_small_m_max(prev)
    assert m.ffn_plan(8, 4096, 2048, 256, 8)["launch_large"] == 0
    with pytest.raises(m.MoeError):
        m.ffn_plan(8, 4096, 2048, 256, 8, 6)


def test_dense_down_cols_setting(lib):
    import mxfp4_mixture_experts_amd as m

    for bad in (-1, 1, 128, 255, 512):
        with pytest.raises(m.MoeError):
            m.set_dense_down_cols(bad)
    prev = m.set_dense_down_cols(224)
    try:
        assert prev == 0
        assert m.set_dense_down_cols(256) == 224
    finally:
        assert m.set_dense_down_cols(prev) == 256


def test_stage_events_validation(lib):
    assert lib.moe_set_stage_events(3, None, None) == -2
    assert lib.moe_set_stage_events(0, None, None) == 0


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
