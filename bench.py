"""Benchmark of the routed MXFP4 MoE layer on one MI355X.

One step = one whole layer (router top-k, grouping, fused gate_up + SwiGLU, down, weighted combine)
on one batch of seeded synthetic input resident in HBM. The default workload is decode at M=8:
T=8 tokens, H=4096, I=2048, E=256 experts, top-8 softmax routing (the c8 decode shape the vllm.cpp
PR #52 node-trace diff measures). Weights are random MXFP4 of that shape, rotated over enough
device replicas that every step streams them cold from HBM (no step finds its weights in the 256 MB
last-level cache). Prints one JSON line: the headline workload's numbers, then the same layer
measurement for the other workloads (one token, two tokens, decode M=2 and M=8 with the unfused
gate/up, per-expert M=1024 on the matrix cores, and the medium (T=256, Zipf-skewed) and high (T=1024)
concurrency batches) under "other_workloads".

  python bench.py [--steps K] [--warmup W] [--config decode_m8] [--mode graph|eager] [--no-others]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, vendor figure
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, vendor figure
LLC_BYTES = 256 << 20           # MI355X Infinity Cache
METRIC = "µs/MoE layer + weight-stream GB/s (% HBM peak) at M=8 decode, 1 GPU"

FP8_MFMA_PEAK_TFLOPS = 5000.0   # MI355X dense fp8 MFMA (also E4M3 x E2M1 on the scaled MFMA)
FP4_MFMA_PEAK_TFLOPS = 10100.0  # MI355X dense fp4 MFMA
# (name, workload, ffn flags, single launch, activation format, from logits) measured after the
# headline, fewer steps each, no CPU baseline. Activation format 1 / 2: the W4A8 / W4A4 FFN
# (moe_mxfp4_ffn_mx). From logits: the layer as one moe_layer_from_logits call.
OTHER_WORKLOADS = (("decode_c1", "decode_c1", 0, False, 0, False), ("decode_m2", "decode_m2", 0, False, 0, False),
                   ("decode_c1_from_logits", "decode_c1", 0, False, 0, True),
                   ("decode_m2_from_logits", "decode_m2", 0, False, 0, True),
                   ("decode_m8_from_logits", "decode_m8", 0, False, 0, True),
                   ("decode_c1_separate_combine", "decode_c1", 8, False, 0, False),
                   ("decode_m2_separate_combine", "decode_m2", 8, False, 0, False),
                   ("decode_m2_unfused", "decode_m2", 1, False, 0, False),
                   ("decode_m8_unfused", "decode_m8", 1, False, 0, False), ("m1024", "m1024", 0, False, 0, False),
                   ("m1024_w4a8", "m1024", 0, False, 1, False), ("m1024_w4a4", "m1024", 0, False, 2, False),
                   ("medium_zipf", "medium_zipf", 0, False, 0, False), ("high_c4", "high_c4", 0, False, 0, False),
                   ("decode_c1_single_launch", "decode_c1", 0, True, 0, False),
                   ("decode_m2_single_launch", "decode_m2", 0, True, 0, False),
                   ("decode_m8_single_launch", "decode_m8", 0, True, 0, False))


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="decode_m8")
    ap.add_argument("--mode", choices=["graph", "eager"], default="graph",
                    help="which timing is reported as value (both are measured)")
    ap.add_argument("--flags", type=int, default=0, help="moe_mxfp4_ffn flags (1 = unfused gate/up, 8 = separate combine launch)")
    ap.add_argument("--act", type=int, default=0, choices=(0, 1, 2),
                    help="headline FFN with MX activations: 1 = W4A8 (MXFP8), 2 = W4A4 (MXFP4)")
    ap.add_argument("--replicas", type=int, default=0, help="weight replicas (0 = enough for cold weights)")
    ap.add_argument("--small-m-max", type=int, default=-1,
                    help="launch-table threshold override (moe_ffn_options.small_m_max; -1 = the library's table)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=3)
    ap.add_argument("--no-others", action="store_true", help="measure the headline workload only")
    ap.add_argument("--single-launch", action="store_true",
                    help="headline through moe_layer_decode (the whole layer in one launch)")
    ap.add_argument("--from-logits", action="store_true",
                    help="headline through moe_layer_from_logits (routing inside the gate_up launch)")
    ap.add_argument("--other-steps", type=int, default=50, help="timed steps of each other workload")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="also run one plain device copy of this many bytes (counter calibration)")
    return ap.parse_args()


# Sources of the weight-streaming kernels (the gate_up stage at decode): the file that defines them and
# the headers it includes. A counter measurement of those kernels stays valid while these are unchanged.
STREAMING_SOURCES = ("common.hpp", "ffn_small.hip", "kernels.hpp", "stream_dev.hpp")


def kernel_source_hash(names=None) -> str:
    """sha256 prefix over the named files of the package's csrc/ (all of them by default)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mxfp4_mixture_experts_amd", "csrc")
    for name in sorted(names if names is not None else os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def committed_traffic(config: str, src_hash: str):
    """HBM traffic per launch of the dominant kernel from the committed counter summary, if it was
    taken on the current kernel sources (otherwise None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_gateup_{config}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.strip().split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha") != src_hash:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def quantile(v, q):
    """q-th decile (1..9) of v, or None for a single value."""
    return round(statistics.quantiles(v, n=10)[q - 1], 2) if len(v) > 1 else None


class Env:
    """torch, the library and the timing stream, shared by every measurement."""

    def __init__(self, args):
        import numpy as np
        import torch

        import moe_synth
        import mxfp4_mixture_experts_amd as moe

        self.np, self.torch, self.moe_synth, self.moe = np, torch, moe_synth, moe
        self.args = args
        self.stream = torch.cuda.Stream()
        torch.cuda.synchronize()

    def event(self):
        return self.torch.cuda.Event(enable_timing=True)

    def dev(self, a):
        return self.torch.from_numpy(self.np.ascontiguousarray(a)).cuda()


def cold_replicas(cfg) -> int:
    """Weight replicas for cold-weight timing. A layer reads only its active experts (at most
    min(E, T*k) of them), so the replicas are counted on those bytes: consecutive layers rotate over
    the replicas, and one full rotation reads at least 8x the 256 MB Infinity Cache, so no layer finds
    its weights there. (Counted on whole replicas, a one-token layer that reads 20 MB of a 0.32 GB
    replica would cycle through 140 MB and run from the cache.)"""
    per_expert = 3 * cfg.H * cfg.I // 2 + 3 * cfg.H * cfg.I // 32
    layer_bytes = min(cfg.E, cfg.T * cfg.k) * per_expert
    return max(2, math.ceil(8 * LLC_BYTES / layer_bytes))


def library_gemm_reference(env, cfg, iters: int = 20) -> dict:
    """Context for the MFMA roofline at large per-expert M: the vendor library's bf16 GEMM (torch.bmm,
    hipBLASLt on ROCm) on the same per-expert shapes as the layer's two GEMMs, with plain bf16
    operands (no FP4 decode), both operands contiguous, timed on the bench stream. Only for
    workloads where every expert holds every token (E == k), so the shapes are exact."""
    torch = env.torch
    E, M, H, I = cfg.E, cfg.T, cfg.H, cfg.I
    out = {"note": "torch.bmm bf16 (hipBLASLt), plain bf16 operands, same per-expert GEMM shapes; "
                   "not part of the layer"}
    g = torch.Generator(device="cuda").manual_seed(0)
    with torch.cuda.stream(env.stream):
        for name, (kdim, ndim) in (("gate_up", (H, 2 * I)), ("down", (I, H))):
            a = torch.randn(E, M, kdim, device="cuda", dtype=torch.bfloat16, generator=g).contiguous()
            b = torch.randn(E, kdim, ndim, device="cuda", dtype=torch.bfloat16, generator=g).contiguous()
            c = torch.empty(E, M, ndim, device="cuda", dtype=torch.bfloat16)
            for _ in range(5):
                torch.bmm(a, b, out=c)
            ev = [env.event() for _ in range(iters + 1)]
            for i in range(iters):
                ev[i].record(env.stream)
                torch.bmm(a, b, out=c)
                ev[i + 1].record(env.stream)
            env.stream.synchronize()
            ts = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(iters))
            flops = 2.0 * E * M * kdim * ndim
            med_us = statistics.median(ts)
            out[name] = {"us_median": round(med_us, 1), "us_min": round(ts[0], 1),
                         "tflops": round(flops / (med_us * 1e-6) / 1e12, 1),
                         "pct_bf16_mfma_peak": round(100 * flops / (med_us * 1e-6) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 1)}
            del a, b, c
    log(f"{cfg.name} library bf16 GEMM reference: gate_up {out['gate_up']['us_median']} us "
        f"({out['gate_up']['tflops']} TFLOP/s), down {out['down']['us_median']} us ({out['down']['tflops']} TFLOP/s)")
    return out


def capture_rotation(torch, stream, L: int, R: int, layer_fn) -> list:
    """hipGraphs of L consecutive layers each, enough of them that replaying them in turn walks over
    all R weight replicas (graph i runs layers i*L .. i*L + L - 1, layer j on replica j mod R)."""
    graphs = []
    for gi in range(max(1, math.ceil(R / L))):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for j in range(L):
                layer_fn((gi * L + j) % R)
        graphs.append(g)
    return graphs


def measure_layer(env: Env, cfg, flags: int, steps: int, warmup: int, small_m_max: int = -1,
                  replicas_override: int = 0, warm: bool = False, single: bool = False, act: int = 0,
                  from_logits: bool = False) -> dict:
    """Eager (per-stage HIP events) and graph (L layers per hipGraph, timed replays) timings of one
    layer workload with cold weights; optionally the warm-weight eager time. `single`: the layer as
    one moe_layer_decode launch (no stages: the launch is the whole layer). `act` 1 / 2: the FFN with
    MXFP8 / MXFP4 activations (moe_mxfp4_ffn_mx). `from_logits`: the layer as one moe_layer_from_logits
    call (stage events as for the FFN; route+group then times what runs before the gate_up launch)."""
    np, torch, moe, moe_synth = env.np, env.torch, env.moe, env.moe_synth
    stream = env.stream
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    t0 = time.time()
    inp = moe_synth.make_inputs(cfg)
    log(f"{cfg.name} flags={flags}: inputs in {time.time() - t0:.1f}s")
    per_expert = 3 * H * I // 2 + 3 * H * I // 32
    replica_bytes = E * per_expert
    R = replicas_override or cold_replicas(cfg)
    first = moe.Mxfp4Weights(*(env.dev(inp[a]) for a in ("w13_q", "w13_s", "w2_q", "w2_s")))
    replicas = [first] + [moe.Mxfp4Weights(*(t.clone() for t in (first.w13_q, first.w13_s, first.w2_q, first.w2_s)))
                          for _ in range(R - 1)]
    x = env.dev(inp["x"].view(np.int16)).view(torch.bfloat16)
    logits = env.dev(inp["logits"])
    layer = moe.MoELayer(first, k, T, cfg.score_fn, cfg.renorm, cfg.clamp, flags, single_launch=single,
                         act_format=act, from_logits=from_logits)
    base_opts = moe.ffn_options(small_m_max=small_m_max)
    torch.cuda.synchronize()
    log(f"{cfg.name}: {R} weight replicas of {replica_bytes / 1e9:.2f} GB on device")

    def step(i, opts=None):
        layer.forward(x, logits, replicas[i % R], stream=stream, options=opts or base_opts)

    with torch.cuda.stream(stream):
        for i in range(warmup):
            step(i)
    torch.cuda.synchronize()
    counts = np.bincount(layer.ids[:T].cpu().numpy().ravel(), minlength=E)
    n_active = int(np.count_nonzero(counts))
    res = dict(cfg=cfg, flags=flags, R=R, inp=inp, n_active=n_active, weight_bytes=n_active * per_expert,
               gateup_bytes=n_active * 2 * I * (H // 2 + H // 32), flops=2 * T * k * 3 * H * I,
               gateup_flops=2 * T * k * 2 * I * H,
               plan=moe.ffn_plan(T, H, I, E, k, flags, base_opts), steps=steps, single=single, act=act,
               from_logits=from_logits,
               routed=from_logits and moe.layer_from_logits_routed(T, H, I, E, k, flags, base_opts))

    # eager: per-step HIP events on the stream the kernels run on: around the whole layer (recorded
    # here) and around the gate_up, down and combine stages (recorded by the library)
    stages = () if single else (moe.STAGE_GATE_UP, moe.STAGE_DOWN, moe.STAGE_COMBINE)
    ev_layer = [(env.event(), env.event()) for _ in range(steps)]
    ev_stage = [[(env.event(), env.event()) for _ in stages] for _ in range(steps)]
    for i in range(steps):  # create the underlying events
        for a, b in [ev_layer[i], *ev_stage[i]]:
            a.record(stream)
            b.record(stream)
    step_opts = [moe.ffn_options(small_m_max=small_m_max, stage_events={st: ev for st, ev in zip(stages, ev_stage[i])})
                 for i in range(steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    with torch.cuda.stream(stream):
        for i in range(steps):
            ev_layer[i][0].record(stream)
            step(i, step_opts[i])
            ev_layer[i][1].record(stream)
    torch.cuda.synchronize()
    res["eager_s"] = time.perf_counter() - t_start
    el = lambda a, b: a.elapsed_time(b) * 1e3  # noqa: E731  (µs)
    res["layer_us"] = [el(*ev_layer[i]) for i in range(steps)]
    med = statistics.median
    if single:
        res["route_group_us"] = res["ffn_us"] = None
        res["stage_us"] = None
        log(f"{cfg.name} single launch eager: {res['eager_s'] / steps * 1e6:.1f} us/layer wall, device median "
            f"{med(res['layer_us']):.1f} us")
    else:
        res["route_group_us"] = [el(ev_layer[i][0], ev_stage[i][0][0]) for i in range(steps)]
        res["ffn_us"] = [el(ev_stage[i][0][0], ev_stage[i][2][1]) for i in range(steps)]
        res["stage_us"] = [[el(*ev_stage[i][j]) for i in range(steps)] for j in range(len(stages))]
        log(f"{cfg.name} eager: {res['eager_s'] / steps * 1e6:.1f} us/layer wall, device median "
            f"{med(res['layer_us']):.1f} us (route+group {med(res['route_group_us']):.1f}, gate_up "
            f"{med(res['stage_us'][0]):.1f}, down {med(res['stage_us'][1]):.1f}, combine {med(res['stage_us'][2]):.1f})")

    # graph: L consecutive layers captured per hipGraph, graphs in turn covering all R replicas;
    # `reps` replays (graph r mod G) with each replay timed; K = reps * L layers in all
    reps = next(r for r in (5, 4, 2, 1) if steps % r == 0 and steps // r >= 2) if steps >= 2 else 1
    L = steps // reps
    res.update(graph_s=None, graph_layer_us=[], L=L, reps=reps)
    try:
        graphs = capture_rotation(torch, stream, L, R, lambda r: layer.forward(x, logits, replicas[r], stream=stream,
                                                                              options=base_opts))
        with torch.cuda.stream(stream):
            for g in graphs:
                g.replay()  # warm-up replays
        torch.cuda.synchronize()
        ev_g = [(env.event(), env.event()) for _ in range(reps)]
        t_start = time.perf_counter()
        with torch.cuda.stream(stream):
            for r_ in range(reps):
                ev_g[r_][0].record(stream)
                graphs[r_ % len(graphs)].replay()
                ev_g[r_][1].record(stream)
        torch.cuda.synchronize()
        res["graph_s"] = time.perf_counter() - t_start
        res["graph_layer_us"] = [el(*ev_g[r_]) / L for r_ in range(reps)]
        log(f"{cfg.name} graph ({L} layers per graph, {reps} replays): median {med(res['graph_layer_us']):.1f} "
            f"us/layer, range {min(res['graph_layer_us']):.1f}-{max(res['graph_layer_us']):.1f}")
        del graphs
    except Exception as exc:  # capture unsupported: report eager
        log(f"graph capture failed: {exc!r}")

    if warm:
        # warm weights, labelled: the same replica every step (what of it fits the 256 MB Infinity
        # Cache stays there), eager, layer events only
        n_warm = min(steps, 50)
        ev_warm = [(env.event(), env.event()) for _ in range(n_warm)]
        with torch.cuda.stream(stream):
            step(0)
            for a, b in ev_warm:
                a.record(stream)
                step(0)
                b.record(stream)
        torch.cuda.synchronize()
        res["warm_us"] = [el(a, b) for a, b in ev_warm]
    res["x"] = x
    del replicas, layer, first
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def roofline_of(res: dict) -> dict:
    """Roofline of the gate_up stage (the dominant kernel: two thirds of the bytes and flops):
    algorithmic weight bytes (HBM-bound decode) or flops (per-expert M = 1024) per launch over its
    mean event-timed duration on the stream it runs on."""
    cfg, plan = res["cfg"], res["plan"]
    if res["single"]:
        # the one launch streams every active expert's weights: all of them over its event-timed mean
        mean_s = statistics.fmean(res["layer_us"]) / 1e6
        achieved = res["weight_bytes"] / mean_s / 1e9
        return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                "kernel": "layer_decode_kernel (route, group, gate_up, down, combine in one launch)",
                "bytes_per_launch": res["weight_bytes"], "avg_launch_us": round(mean_s * 1e6, 2)}
    gateup_mean_s = statistics.fmean(res["stage_us"][0]) / 1e6
    if res["act"]:
        peak = FP8_MFMA_PEAK_TFLOPS if res["act"] == 1 else FP4_MFMA_PEAK_TFLOPS
        achieved = res["gateup_flops"] / gateup_mean_s / 1e12
        return {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": None,
                "kernel": "mx_gemm_kernel gate_up (block-scaled MFMA, " +
                          ("E4M3" if res["act"] == 1 else "E2M1") + " activations x E2M1 weights)",
                "flops_per_launch": res["gateup_flops"], "avg_launch_us": round(gateup_mean_s * 1e6, 2)}
    large = plan["launch_large"]
    mfma_bound = cfg.name == "m1024"
    if mfma_bound:
        achieved = res["gateup_flops"] / gateup_mean_s / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / BF16_MFMA_PEAK_TFLOPS, 4), "traffic": None}
    else:
        achieved = res["gateup_bytes"] / gateup_mean_s / 1e9
        # the counters were taken on the fused weight-streaming kernel; with MFMA kernels in the stage
        # too the measurement must match every source
        traffic = None if res["flags"] else committed_traffic(
            cfg.name, kernel_source_hash(None if large else STREAMING_SOURCES))
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic}
    roofline["kernel"] = "gate_up stage (" + (
        "weight-streaming + MFMA kernels" if large and plan["launch_small"] else
        "dense MFMA kernel" if large else "weight-streaming kernel" +
        (", gate and up passes" if res["flags"] & 1 else "")) + ")"
    roofline["bytes_per_launch" if not mfma_bound else "flops_per_launch"] = (
        res["gateup_bytes"] if not mfma_bound else res["gateup_flops"])
    roofline["avg_launch_us"] = round(gateup_mean_s * 1e6, 2)
    return roofline


def workload_name(cfg) -> str:
    return (f"{cfg.name}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} top-{cfg.k} "
            f"{'sigmoid' if cfg.score_fn else 'softmax'} renorm" + (f", clamp {cfg.clamp}" if cfg.clamp else ""))


def summary(res: dict, use_graph: bool) -> dict:
    """The per-workload numbers every measured workload reports."""
    med = statistics.median
    use_graph = use_graph and bool(res["graph_layer_us"])
    us_layer = med(res["graph_layer_us"]) if use_graph else med(res["layer_us"])
    gbps = res["weight_bytes"] / (us_layer * 1e-6) / 1e9
    tflops = res["flops"] / (us_layer * 1e-6) / 1e12
    stage = res["stage_us"]
    if res["single"]:
        stages = None
        ffn_only = None
    else:
        stages = {"route+group": round(med(res["route_group_us"]), 2), "gate_up": round(med(stage[0]), 2),
                  "down": round(med(stage[1]), 2), "combine": round(med(stage[2]), 2)}
        ffn_only = round(med(res["ffn_us"]), 2)
    return {
        "us_per_layer": round(us_layer, 2),
        "timing": (f"hipGraph of {res['L']} layers, median of {res['reps']} replays" if use_graph
                   else "eager, median step"),
        "weight_stream_GBps": round(gbps, 1),
        "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 1),
        "tflops": round(tflops, 2),
        "pct_bf16_mfma_peak": round(100 * tflops / BF16_MFMA_PEAK_TFLOPS, 1),
        "ffn_only_us": ffn_only,
        "stage_us_eager_median": stages,
        "us_per_layer_eager": {"median": round(med(res["layer_us"]), 2), "p10": quantile(res["layer_us"], 1),
                               "p90": quantile(res["layer_us"], 9),
                               "host_wall": round(res["eager_s"] / res["steps"] * 1e6, 2)},
        "us_per_layer_graph": ({"median": round(med(res["graph_layer_us"]), 2),
                                "min": round(min(res["graph_layer_us"]), 2),
                                "max": round(max(res["graph_layer_us"]), 2)} if res["graph_layer_us"] else None),
        "active_experts": res["n_active"],
        "weight_bytes_per_layer": res["weight_bytes"],
        "flops_per_layer": res["flops"],
        "roofline": roofline_of(res),
        "config": {"workload": workload_name(res["cfg"]), "flags": res["flags"], "weight_replicas": res["R"],
                   "small_m_max": res["plan"]["small_m_max"],
                   "path": "moe_layer_decode (one launch)" if res["single"] else
                           ("moe_layer_from_logits (" + ("routing and grouping inside the gate_up launch)"
                                                         if res["routed"] else "routing launch first)"))
                           if res["from_logits"] else
                           ("moe_route_group + moe_mxfp4_ffn_mx (" + ("W4A8: MXFP8" if res["act"] == 1 else
                                                                      "W4A4: MXFP4") + " activations)")
                           if res["act"] else "moe_route_group + moe_mxfp4_ffn (multi-launch)"},
    }


def forward_timing(env: Env, cfg, steps: int) -> dict | None:
    """The layer from the activations and the router weights (moe_layer_forward: the router, its
    selection and the grouping, then the FFN): one hipGraph of L layers on cold expert weights (the
    same rotation as the headline), median over timed replays. Not part of `value`, which starts
    from logits as the metric's layer does."""
    np, torch, moe, moe_synth = env.np, env.torch, env.moe, env.moe_synth
    stream = env.stream
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    inp = moe_synth.make_inputs(cfg)
    R = cold_replicas(cfg)
    first = moe.Mxfp4Weights(*(env.dev(inp[a]) for a in ("w13_q", "w13_s", "w2_q", "w2_s")))
    replicas = [first] + [moe.Mxfp4Weights(*(t.clone() for t in (first.w13_q, first.w13_s, first.w2_q, first.w2_s)))
                          for _ in range(R - 1)]
    x = env.dev(inp["x"].view(np.int16)).view(torch.bfloat16)
    wr = env.dev(moe_synth.make_router_weights(E, H, 20261203 + 99).view(np.int16)).view(torch.bfloat16)
    ws = moe.layer_forward_workspace(T, H, I, E, k)
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    fwd = lambda j: moe.layer_forward(x, wr, replicas[j % R], k, cfg.score_fn, cfg.renorm, cfg.clamp,  # noqa: E731
                                      out=out, workspace=ws, stream=stream)
    try:
        with torch.cuda.stream(stream):
            for j in range(5):
                fwd(j)
        torch.cuda.synchronize()
        reps = 5
        L = max(2, steps // reps)
        graphs = capture_rotation(torch, stream, L, R, fwd)
        with torch.cuda.stream(stream):
            for g in graphs:
                g.replay()
        torch.cuda.synchronize()
        times = []
        for r_ in range(reps):
            a, b = env.event(), env.event()
            with torch.cuda.stream(stream):
                a.record(stream)
                graphs[r_ % len(graphs)].replay()
                b.record(stream)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) * 1e3 / L)
        del graphs
    except Exception as exc:  # capture unsupported
        log(f"layer_forward graph failed: {exc!r}")
        return None
    finally:
        del replicas, first
        torch.cuda.empty_cache()
    us = statistics.median(times)
    log(f"layer_forward (from x and W_router) {cfg.name}: {us:.1f} us/layer")
    return {"us_per_layer": round(us, 2), "timing": f"hipGraph of {L} layers, median of {reps} replays",
            "note": "x and bf16 W_router [E, H] to out: router projection + top-k + grouping (one launch up to "
                    "32 tokens), gate_up, down, combine; cold expert weights; not part of value"}


def read_probe_gbps(env: Env) -> float:
    """Attainable read bandwidth on this machine: a plain device reduction of 2 GiB in rows of 4096
    floats (one output per row; best of 5). A single whole-buffer sum reaches only about two thirds
    of it."""
    torch = env.torch
    probe = torch.zeros((1 << 31) // 4, dtype=torch.float32, device="cuda")
    probe_s = []
    for _ in range(5):
        a, b = env.event(), env.event()
        a.record(env.stream)
        with torch.cuda.stream(env.stream):
            probe.view(-1, 4096).sum(dim=1)
        b.record(env.stream)
        torch.cuda.synchronize()
        probe_s.append(a.elapsed_time(b) / 1e3)
    v = probe.numel() * 4 / min(probe_s) / 1e9
    del probe
    torch.cuda.empty_cache()
    return v


def router_timing(env: Env, cfg, x) -> dict | None:
    """The router projection + top-k at this workload's sizes (the step before routing; not part of
    `value`): bf16 W_router[E, H]; one hipGraph over enough copies of (W_router, x) that every call
    reads cold operands (four times the Infinity Cache in total: at twice it, a cyclic sweep still
    found some of its operands there), best of 5 replays."""
    np, torch, moe, moe_synth = env.np, env.torch, env.moe, env.moe_synth
    stream = env.stream
    T, H, E, k = cfg.T, cfg.H, cfg.E, cfg.k
    router_bytes = E * H * 2 + T * H * 2
    n_router = max(8, min(1024, math.ceil(4 * LLC_BYTES / router_bytes)))
    w_router0 = env.dev(moe_synth.make_router_weights(E, H, 20261203 + 99).view(np.int16)).view(torch.bfloat16)
    r_ops = [(w_router0.clone(), x.clone()) for _ in range(n_router)]
    del w_router0
    ws_router = moe.router_workspace(T, H, E)
    with torch.cuda.stream(stream):
        moe.router_gemm_topk(r_ops[0][1], r_ops[0][0], k, cfg.score_fn, cfg.renorm, want_logits=False,
                             workspace=ws_router, stream=stream)
    torch.cuda.synchronize()

    def graph_us(ops):
        """Per-call time of one hipGraph of calls over `ops`, best of 5 replays on `stream`."""
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=stream):
            for wr_i, xr_i in ops:
                moe.router_gemm_topk(xr_i, wr_i, k, cfg.score_fn, cfg.renorm, want_logits=False,
                                     workspace=ws_router, stream=stream, split_launch=split[0])
        with torch.cuda.stream(stream):  # a replay runs on the current stream: make it `stream`
            gr.replay()
        torch.cuda.synchronize()
        best = None
        for _ in range(5):
            a, b = env.event(), env.event()
            with torch.cuda.stream(stream):
                a.record(stream)
                gr.replay()
                b.record(stream)
            torch.cuda.synchronize()
            v = a.elapsed_time(b) * 1e3 / len(ops)
            best = v if best is None else min(best, v)
        del gr
        return best

    split = [False]

    def graph_us_split(ops):
        split[0] = True
        try:
            return graph_us(ops)
        finally:
            split[0] = False

    try:
        us = graph_us(r_ops)
        us_warm = graph_us([r_ops[0]] * 50)
        us_two = graph_us_split(r_ops)
    except Exception as exc:  # capture unsupported: skip the router line
        log(f"router graph capture failed: {exc!r}")
        return None
    finally:
        del r_ops
        torch.cuda.empty_cache()
    log(f"router gemm+top-k: {us:.2f} us per call cold ({n_router} operand copies), {us_warm:.2f} us warm, "
        f"{us_two:.2f} us cold as two launches")
    return {
        "us": round(us, 2),
        "operand_GBps": round(router_bytes / (us * 1e-6) / 1e9, 1),
        "pct_hbm_peak": round(100 * router_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 1),
        "tflops": round(2 * T * E * H / (us * 1e-6) / 1e12, 2),
        "us_warm": round(us_warm, 2),
        "us_two_launches": round(us_two, 2),
        "note": (f"logits = x . W_router^T (bf16 [E, H]) and top-k; us: one graph over {n_router} copies of "
                 "(W_router, x), so every call reads cold operands (GB/s counts W_router and x once); "
                 "us_warm: 50 calls on one copy; us_two_launches: cold, the projection and the selection as "
                 "two kernels (one launch is the default up to 32 tokens); not part of value")}


def cpu_baseline(args, cfg, inp) -> dict:
    """The oracle, as it stands, on the host cores: a bounded sample of the workload's tokens,
    scaled to the whole layer."""
    import oracle

    host_cores = os.cpu_count() or 1
    threads = min(16, host_cores)
    times = []
    sample_tokens = cfg.T if cfg.T <= 8 else 1
    for rep in range(args.cpu_reps):
        t_c = time.perf_counter()
        oracle.moe_layer(inp["logits"][:sample_tokens], inp["x"][:sample_tokens], inp["w13_q"], inp["w13_s"],
                         inp["w2_q"], inp["w2_s"], cfg.k, cfg.score_fn, cfg.renorm, cfg.clamp, threads)
        times.append(time.perf_counter() - t_c)
        log(f"oracle rep {rep}: {times[-1]:.2f}s")
    per_layer_us = statistics.median(times) * 1e6 * (cfg.T / sample_tokens)
    used = oracle.num_threads(threads)
    # one thread, on one token (a layer's cost is proportional to its routed pairs), once
    t_c = time.perf_counter()
    oracle.moe_layer(inp["logits"][:1], inp["x"][:1], inp["w13_q"], inp["w13_s"], inp["w2_q"], inp["w2_s"], cfg.k,
                     cfg.score_fn, cfg.renorm, cfg.clamp, 1)
    one_us = (time.perf_counter() - t_c) * 1e6 * cfg.T
    log(f"oracle, one thread, one token: {one_us / cfg.T / 1e6:.2f}s")
    return {"value": round(per_layer_us, 1), "unit": "µs/layer", "cores": used, "kind": "oracle",
            "threads_used": used, "host_cores": host_cores,
            "sample": (f"{sample_tokens} of {cfg.T} tokens of one {cfg.name} layer (route+group+ffn+combine, "
                       f"fp64, {used} OpenMP threads on a host reporting {host_cores} cores), median of "
                       f"{args.cpu_reps}, scaled to the whole layer"),
            "single_thread": {"value": round(one_us, 1), "unit": "µs/layer", "threads_used": 1,
                              "sample": f"1 of {cfg.T} tokens, one run, scaled to the whole layer"}}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the layer would shard by "
              "experts or by the intermediate dimension, with one all-to-all or all-reduce per layer); "
              "run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    env = Env(args)
    env.moe.load_library()
    cfg = env.moe_synth.CONFIGS[args.config]

    res = measure_layer(env, cfg, args.flags, args.steps, args.warmup, args.small_m_max, args.replicas, warm=True,
                        single=args.single_launch, act=args.act, from_logits=args.from_logits)
    if args.copy_bytes:
        src = torch.empty(args.copy_bytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy of {args.copy_bytes} bytes done")
        del src, dst
    probe = read_probe_gbps(env)
    med = statistics.median
    log(f"warm weights: median {med(res['warm_us']):.1f} us/layer eager; read probe {probe:.0f} GB/s")
    router = router_timing(env, cfg, res["x"])
    forward = (forward_timing(env, cfg, args.steps) if args.flags == 0 and not args.single_launch and not args.act
               else None)

    use_graph = args.mode == "graph" and res["graph_s"] is not None
    s = summary(res, use_graph)
    us_layer = s["us_per_layer"]
    gbps = s["weight_stream_GBps"]
    cpu = None if args.no_cpu_baseline else cpu_baseline(args, cfg, res["inp"])

    others = {}
    if not args.no_others:
        for name, wl, flags, single, act, lg in OTHER_WORKLOADS:
            if (wl == cfg.name and flags == args.flags and single == args.single_launch and act == args.act
                    and lg == args.from_logits):
                continue
            o = measure_layer(env, env.moe_synth.CONFIGS[wl], flags, args.other_steps, max(5, args.warmup // 2),
                              single=single, act=act, from_logits=lg)
            others[name] = summary(o, True)
            others[name]["steps"] = args.other_steps
            del o
            if name == "m1024":
                others[name]["library_bf16_gemm"] = library_gemm_reference(env, env.moe_synth.CONFIGS[wl])

    rec = {
        "metric": METRIC,
        "value": us_layer,
        "unit": "µs/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_layer / 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4 weights, bf16 activations, fp32 accumulate",
        "data": "synthetic (seeded; random MXFP4 weights, no checkpoint)",
        "config": {"workload": workload_name(cfg), "timing": s["timing"], "flags": args.flags,
                   "path": s["config"]["path"],
                   "weight_replicas": res["R"], "parallelism": "none (1 GPU)",
                   "small_m_max": res["plan"]["small_m_max"]},
        "weight_stream_GBps": gbps,
        "pct_hbm_peak": s["pct_hbm_peak"],
        "ffn_only_us": s["ffn_only_us"],
        "weight_stream_GBps_ffn_only": (round(res["weight_bytes"] / (s["ffn_only_us"] * 1e-6) / 1e9, 1)
                                        if s["ffn_only_us"] else None),
        "read_probe_GBps": round(probe, 1),
        "pct_read_probe": round(100 * gbps / probe, 1),
        "us_per_layer_warm_eager": {"median": round(med(res["warm_us"]), 2), "steps": len(res["warm_us"]),
                                    "note": "one weight replica reused every step (not the metric)"},
        "router_gemm_topk": router,
        "layer_forward_from_x": forward,
        "stage_us_eager_median": s["stage_us_eager_median"],
        "active_experts": res["n_active"],
        "weight_bytes_per_layer": res["weight_bytes"],
        "tflops": s["tflops"],
        "us_per_layer_eager": s["us_per_layer_eager"],
        "us_per_layer_graph": s["us_per_layer_graph"],
        "roofline": s["roofline"],
        "cpu_baseline": cpu,
        "other_workloads": others,
        "kernel_source_sha": kernel_source_hash(),
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
