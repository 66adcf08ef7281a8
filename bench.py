"""Benchmark of the routed MXFP4 MoE layer on one MI355X.

One step = one whole layer (router top-k, grouping, fused gate_up + SwiGLU, down, weighted combine)
on one batch of seeded synthetic input resident in HBM. The default workload is decode at M=8:
T=8 tokens, H=4096, I=2048, E=256 experts, top-8 softmax routing (the c8 decode shape the vllm.cpp
PR #52 node-trace diff measures). Weights are random MXFP4 of that shape, rotated over enough
device replicas that every step streams them cold from HBM (no step finds its weights in the 256 MB
last-level cache). Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--config decode_m8] [--mode graph|eager]
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
    ap.add_argument("--flags", type=int, default=0, help="moe_mxfp4_ffn flags (1 = unfused gate/up)")
    ap.add_argument("--replicas", type=int, default=0, help="weight replicas (0 = enough for cold weights)")
    ap.add_argument("--small-m-max", type=int, default=-1,
                    help="launch-table threshold override (moe_ffn_options.small_m_max; -1 = the library's table)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=3)
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="also run one plain device copy of this many bytes (counter calibration)")
    return ap.parse_args()


# Sources of the weight-streaming kernels (the gate_up stage at decode): the file that defines them and
# the headers it includes. A counter measurement of those kernels stays valid while these are unchanged.
STREAMING_SOURCES = ("common.hpp", "ffn_small.hip", "kernels.hpp")


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


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the layer would shard by "
              "experts or by the intermediate dimension, with one all-to-all or all-reduce per layer); "
              "run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import moe_synth
    import mxfp4_mixture_experts_amd as moe

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    moe.load_library()
    base_opts = moe.ffn_options(small_m_max=args.small_m_max)
    cfg = moe_synth.CONFIGS[args.config]
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    t0 = time.time()
    inp = moe_synth.make_inputs(cfg)
    log(f"generated {cfg.name} inputs in {time.time() - t0:.1f}s")

    per_expert = 3 * H * I // 2 + 3 * H * I // 32
    replica_bytes = E * per_expert
    R = args.replicas or max(2, math.ceil((2 << 30) / replica_bytes), math.ceil(8 * LLC_BYTES / replica_bytes))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    host = [inp["w13_q"], inp["w13_s"], inp["w2_q"], inp["w2_s"]]
    first = moe.Mxfp4Weights(*(dev(a) for a in host))
    replicas = [first] + [moe.Mxfp4Weights(*(t.clone() for t in (first.w13_q, first.w13_s, first.w2_q, first.w2_s)))
                          for _ in range(R - 1)]
    del host
    x = dev(inp["x"].view(np.int16)).view(torch.bfloat16)
    logits = dev(inp["logits"])
    layer = moe.MoELayer(first, k, T, cfg.score_fn, cfg.renorm, cfg.clamp, args.flags)
    torch.cuda.synchronize()
    log(f"{R} weight replicas of {replica_bytes / 1e9:.2f} GB on device")

    stream = torch.cuda.Stream()
    torch.cuda.synchronize()

    def step(i, opts=None):
        layer.forward(x, logits, replicas[i % R], stream=stream, options=opts or base_opts)

    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
    torch.cuda.synchronize()
    counts = layer.grp.counts.cpu().numpy()
    n_active = int(np.count_nonzero(counts))
    weight_bytes = n_active * per_expert
    gateup_bytes = n_active * 2 * I * (H // 2 + H // 32)
    flops = 2 * T * k * 3 * H * I
    gateup_flops = 2 * T * k * 2 * I * H

    if args.copy_bytes:
        src = torch.empty(args.copy_bytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy of {args.copy_bytes} bytes done")

    # eager: per-step HIP events on the stream the kernels run on: around the whole layer (recorded
    # here) and around the gate_up, down and combine stages (recorded by the library)
    stages = (moe.STAGE_GATE_UP, moe.STAGE_DOWN, moe.STAGE_COMBINE)
    mk = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    ev_layer = [(mk(), mk()) for _ in range(args.steps)]
    ev_stage = [[(mk(), mk()) for _ in stages] for _ in range(args.steps)]
    for i in range(args.steps):  # create the underlying events
        for a, b in [ev_layer[i], *ev_stage[i]]:
            a.record(stream)
            b.record(stream)
    torch.cuda.synchronize()
    step_opts = [moe.ffn_options(small_m_max=args.small_m_max,
                                 stage_events={st: ev for st, ev in zip(stages, ev_stage[i])})
                 for i in range(args.steps)]
    t_start = time.perf_counter()
    with torch.cuda.stream(stream):
        for i in range(args.steps):
            ev_layer[i][0].record(stream)
            step(i, step_opts[i])
            ev_layer[i][1].record(stream)
    torch.cuda.synchronize()
    eager_s = time.perf_counter() - t_start
    el = lambda a, b: a.elapsed_time(b) * 1e3  # noqa: E731  (µs)
    layer_us = [el(*ev_layer[i]) for i in range(args.steps)]
    route_group_us = [el(ev_layer[i][0], ev_stage[i][0][0]) for i in range(args.steps)]
    ffn_us = [el(ev_stage[i][0][0], ev_stage[i][2][1]) for i in range(args.steps)]
    stage_us = [[el(*ev_stage[i][j]) for i in range(args.steps)] for j in range(len(stages))]
    gateup_mean_s = statistics.fmean(stage_us[0]) / 1e6
    med = statistics.median
    log(f"eager: {eager_s / args.steps * 1e6:.1f} us/layer wall, device median {med(layer_us):.1f} us "
        f"(route+group {med(route_group_us):.1f}, gate_up {med(stage_us[0]):.1f}, down {med(stage_us[1]):.1f}, "
        f"combine {med(stage_us[2]):.1f})")

    # graph: L consecutive layers captured in one hipGraph (layer j on replica j mod R), replayed
    # `reps` times with each replay timed; K = reps * L layers in all
    reps = next(r for r in (5, 4, 2, 1) if args.steps % r == 0 and args.steps // r >= 2) if args.steps >= 2 else 1
    L = args.steps // reps
    graph_s = None
    graph_layer_us = []
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for j in range(L):
                layer.forward(x, logits, replicas[j % R], stream=stream, options=base_opts)
        g.replay()  # warm-up replay
        torch.cuda.synchronize()
        ev_g = [(mk(), mk()) for _ in range(reps)]
        t_start = time.perf_counter()
        with torch.cuda.stream(stream):
            for r_ in range(reps):
                ev_g[r_][0].record(stream)
                g.replay()
                ev_g[r_][1].record(stream)
        torch.cuda.synchronize()
        graph_s = time.perf_counter() - t_start
        graph_layer_us = [el(*ev_g[r_]) / L for r_ in range(reps)]
        log(f"graph ({L} layers per graph, {reps} replays): median {med(graph_layer_us):.1f} us/layer, "
            f"range {min(graph_layer_us):.1f}-{max(graph_layer_us):.1f}")
        del g
    except Exception as exc:  # capture unsupported: report eager
        log(f"graph capture failed: {exc!r}")

    # warm weights, labelled: the same replica every step (what of it fits the 256 MB Infinity Cache
    # stays there), eager, layer events only
    n_warm = min(args.steps, 50)
    ev_warm = [(mk(), mk()) for _ in range(n_warm)]
    with torch.cuda.stream(stream):
        step(0)
        for a, b in ev_warm:
            a.record(stream)
            step(0)
            b.record(stream)
    torch.cuda.synchronize()
    warm_us = [el(a, b) for a, b in ev_warm]

    # attainable read bandwidth on this machine: a plain device reduction of 2 GiB in rows of 4096 floats
    # (one output per row; best of 5). A single whole-buffer sum reaches only about two thirds of it.
    probe = torch.zeros((1 << 31) // 4, dtype=torch.float32, device="cuda")
    probe_s = []
    for _ in range(5):
        a, b = mk(), mk()
        a.record(stream)
        with torch.cuda.stream(stream):
            probe.view(-1, 4096).sum(dim=1)
        b.record(stream)
        torch.cuda.synchronize()
        probe_s.append(a.elapsed_time(b) / 1e3)
    read_probe_gbps = probe.numel() * 4 / min(probe_s) / 1e9
    del probe
    log(f"warm weights: median {med(warm_us):.1f} us/layer eager; read probe {read_probe_gbps:.0f} GB/s")

    # the router projection + top-k at this workload's sizes (the step before routing; not part of
    # `value`): bf16 W_router[E, H]; one hipGraph over enough copies of (W_router, x) that every call
    # reads cold operands (four times the Infinity Cache in total: at twice it, a cyclic sweep still
    # found some of its operands there), best of 5 replays
    router_bytes = E * H * 2 + T * H * 2
    n_router = max(8, min(1024, math.ceil(4 * LLC_BYTES / router_bytes)))
    w_router0 = dev(moe_synth.make_router_weights(E, H, 20261203 + 99).view(np.int16)).view(torch.bfloat16)
    r_ops = [(w_router0.clone(), x.clone()) for _ in range(n_router)]
    del w_router0
    ws_router = torch.empty(moe.router_gemm_topk_workspace_size(T, H, E), dtype=torch.uint8, device="cuda")
    with torch.cuda.stream(stream):
        moe.router_gemm_topk(r_ops[0][1], r_ops[0][0], k, cfg.score_fn, cfg.renorm, want_logits=False,
                             workspace=ws_router, stream=stream)
    torch.cuda.synchronize()

    def router_graph_us(ops):
        """Per-call time of one hipGraph of calls over `ops`, best of 5 replays on `stream`."""
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=stream):
            for wr_i, xr_i in ops:
                moe.router_gemm_topk(xr_i, wr_i, k, cfg.score_fn, cfg.renorm, want_logits=False,
                                     workspace=ws_router, stream=stream)
        with torch.cuda.stream(stream):  # a replay runs on the current stream: make it `stream`
            gr.replay()
        torch.cuda.synchronize()
        best = None
        for _ in range(5):
            a, b = mk(), mk()
            with torch.cuda.stream(stream):
                a.record(stream)
                gr.replay()
                b.record(stream)
            torch.cuda.synchronize()
            v = a.elapsed_time(b) * 1e3 / len(ops)
            best = v if best is None else min(best, v)
        del gr
        return best

    router_us = router_warm_us = None
    try:
        router_us = router_graph_us(r_ops)
        router_warm_us = router_graph_us([r_ops[0]] * 50)
    except Exception as exc:  # capture unsupported: skip the router line
        log(f"router graph capture failed: {exc!r}")
    del r_ops
    if router_us is not None:
        log(f"router gemm+top-k: {router_us:.2f} us per call cold ({n_router} operand copies), "
            f"{router_warm_us:.2f} us warm")

    use_graph = args.mode == "graph" and graph_s is not None
    total_s = graph_s if use_graph else eager_s
    us_layer = med(graph_layer_us) if use_graph else med(layer_us)
    gbps = weight_bytes / (us_layer * 1e-6) / 1e9
    ffn_med = med(ffn_us)

    plan = moe.ffn_plan(T, H, I, E, k, args.flags, base_opts)
    large = plan["launch_large"]
    mfma_bound = cfg.name == "m1024"
    if mfma_bound:
        achieved = gateup_flops / gateup_mean_s / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / BF16_MFMA_PEAK_TFLOPS, 4), "traffic": None}
    else:
        achieved = gateup_bytes / gateup_mean_s / 1e9
        # the counters were taken on the weight-streaming kernel; with MFMA kernels in the stage too
        # the measurement must match every source
        traffic = committed_traffic(cfg.name, kernel_source_hash(None if large else STREAMING_SOURCES))
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic}
    roofline["kernel"] = "gate_up stage (" + (
        "weight-streaming + MFMA kernels" if large and plan["launch_small"] else "MFMA kernel" if large
        else "weight-streaming kernel") + ")"
    roofline["bytes_per_launch" if not mfma_bound else "flops_per_launch"] = (
        gateup_bytes if not mfma_bound else gateup_flops)
    roofline["avg_launch_us"] = round(gateup_mean_s * 1e6, 2)

    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        threads = min(16, os.cpu_count() or 1)
        times = []
        sample_tokens = T if cfg.T <= 8 else 1
        for rep in range(args.cpu_reps):
            t_c = time.perf_counter()
            oracle.moe_layer(inp["logits"][:sample_tokens], inp["x"][:sample_tokens], inp["w13_q"], inp["w13_s"],
                             inp["w2_q"], inp["w2_s"], k, cfg.score_fn, cfg.renorm, cfg.clamp, threads)
            times.append(time.perf_counter() - t_c)
            log(f"oracle rep {rep}: {times[-1]:.2f}s")
        per_layer_us = statistics.median(times) * 1e6 * (T / sample_tokens)
        cpu = {"value": round(per_layer_us, 1), "unit": "µs/layer", "cores": oracle.num_threads(threads),
               "kind": "oracle",
               "sample": (f"{sample_tokens} of {T} tokens of one {cfg.name} layer (route+group+ffn+combine, "
                          f"fp64), median of {args.cpu_reps}, scaled to the whole layer")}

    rec = {
        "metric": METRIC,
        "value": round(us_layer, 2),
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
        "config": {"workload": f"{cfg.name}: T={T} H={H} I={I} E={E} top-{k} "
                               f"{'sigmoid' if cfg.score_fn else 'softmax'} renorm"
                               + (f", clamp {cfg.clamp}" if cfg.clamp else ""),
                   "timing": (f"hipGraph of {L} layers, median of {reps} replays" if use_graph
                              else "eager, median step"),
                   "flags": args.flags, "weight_replicas": R, "parallelism": "none (1 GPU)",
                   "small_m_max": plan["small_m_max"]},
        "weight_stream_GBps": round(gbps, 1),
        "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 1),
        "ffn_only_us": round(ffn_med, 2),
        "weight_stream_GBps_ffn_only": round(weight_bytes / (ffn_med * 1e-6) / 1e9, 1),
        "read_probe_GBps": round(read_probe_gbps, 1),
        "pct_read_probe": round(100 * gbps / read_probe_gbps, 1),
        "us_per_layer_warm_eager": {"median": round(med(warm_us), 2), "steps": n_warm,
                                    "note": "one weight replica reused every step (not the metric)"},
        "router_gemm_topk": (None if router_us is None else {
            "us": round(router_us, 2),
            "operand_GBps": round(router_bytes / (router_us * 1e-6) / 1e9, 1),
            "pct_hbm_peak": round(100 * router_bytes / (router_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 1),
            "tflops": round(2 * T * E * H / (router_us * 1e-6) / 1e12, 2),
            "us_warm": round(router_warm_us, 2),
            "note": (f"logits = x . W_router^T (bf16 [E, H]) and top-k; us: one graph over {n_router} copies of "
                     "(W_router, x), so every call reads cold operands (GB/s counts W_router and x once); "
                     "us_warm: 50 calls on one copy; not part of value")}),
        "stage_us_eager_median": {"route+group": round(med(route_group_us), 2), "gate_up": round(med(stage_us[0]), 2),
                                  "down": round(med(stage_us[1]), 2), "combine": round(med(stage_us[2]), 2)},
        "active_experts": n_active,
        "weight_bytes_per_layer": weight_bytes,
        "tflops": round(flops / (us_layer * 1e-6) / 1e12, 2),
        "us_per_layer_eager": {"median": round(med(layer_us), 2),
                               "p10": round(statistics.quantiles(layer_us, n=10)[0], 2) if len(layer_us) > 1 else None,
                               "p90": round(statistics.quantiles(layer_us, n=10)[-1], 2) if len(layer_us) > 1 else None,
                               "host_wall": round(eager_s / args.steps * 1e6, 2)},
        "us_per_layer_graph": ({"median": round(med(graph_layer_us), 2), "min": round(min(graph_layer_us), 2),
                                "max": round(max(graph_layer_us), 2)} if graph_layer_us else None),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernel_source_sha": kernel_source_hash(),
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
