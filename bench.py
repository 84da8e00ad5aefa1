"""Decode MoE layer benchmark on one MI355X.

Workload (default): Qwen3-30B-A3B-shaped MoE layer -- H=2048, N=128 experts,
top-8, expert intermediate 768, bf16 experts (9.44 MB each), router W_r fp32
[128, 2048] -- at B=16 decode tokens, x ~ N(0,1) bf16, weights ~ N(0, 0.02).
One step = one pass of the whole layer on one batch: router logits -> OEA
(simplified, k0=3) routing -> dispatch -> expert FFN with weighted combine.
Steps rotate over 8 device copies of the layer and 10 batches, so successive
steps read different weight memory (as successive decoder layers do) and the
256 MB last-level cache cannot serve them.  Vanilla top-8 and OEA k0=5 are
timed the same way and reported beside it.

value = whole-layer algorithmic bytes / layer time, in GB/s, where bytes =
sum over active experts of their weight bytes + router weights + x + y.
The roofline entry is the expert FFN (the dominant work): its algorithmic
bytes per call (active-expert weights + x + y) over its average duration,
timed with HIP events on the stream it is launched on.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "MoE-layer decode µs & HBM GB/s (% peak) vs unique experts T, top-8 vs OEA"


_T0 = time.time()


def progress(msg: str) -> None:
    """One progress line on stderr (the JSON result goes to stdout)."""
    print(f"bench [{time.time() - _T0:6.1f} s] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="qwen30b", choices=["qwen30b", "qwen235b"])
    ap.add_argument("--batch", type=int, default=16)
    ap.add_argument("--k0", type=int, default=3)
    ap.add_argument("--copies", type=int, default=8)
    ap.add_argument("--batches", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--only", choices=["oea", "topk", "mixed", "point"], default=None,
                    help="time only this routing, only the mixed bf16/INT4 layer at B=32, or only one "
                         "batch-sweep point (--batch, --routing, --k0, --zipf) (for profiler runs)")
    ap.add_argument("--routing", choices=["oea", "topk"], default="oea", help="routing of --only point")
    ap.add_argument("--zipf", type=float, default=1.1, help="Zipf bias exponent of --only point (0: uniform)")
    ap.add_argument("--no-extended", action="store_true",
                    help="skip the batch sweep, the 235B-shaped layer and the mixed INT4 layer")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run 20 plain device copies of MIB MiB (the "
                         "reference kernel for scaling HBM byte counters) and exit")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "expert_ffn_traffic_qwen30b_b16_oea3.txt")
FFN_SOURCES = [os.path.join(ROOT, "aware_expert_routing_amd", "csrc", f) for f in ("ffn.hip", "pack.hip")]


def sources_sha256():
    """Hash of the expert-FFN sources with comments and whitespace removed,
    so that the counters stay attached to the code they were taken on."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in FFN_SOURCES:
        with open(f) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def measured_traffic(prefix=""):
    """HBM bytes per expert-FFN call (prefix "") or per phase-A launch (prefix
    "phase_a_") from the committed counter summary, or None when it is missing
    or was taken on different kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.lstrip().startswith("#"):
            key, val = line.split("=", 1)
            kv[key.strip()] = val.strip()
    if kv.get("sources_sha256") != sources_sha256():
        return None
    try:
        return int(float(kv[prefix + "fetch_bytes_per_call"]) + float(kv[prefix + "write_bytes_per_call"]))
    except (KeyError, ValueError):
        return None


def copy_calibration(mib):
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, device="cuda:0", dtype=torch.float32)
    dst = torch.empty_like(src)
    for _ in range(20):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read_per_copy": n * 4, "bytes_written_per_copy": n * 4,
                                           "copies": 20}}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import numpy as np
    import torch

    import aware_expert_routing_amd as moe
    import synth

    t_setup = time.time()
    dev = torch.device("cuda:0")
    shape = synth.SHAPES[args.config]
    N, k, H, I = shape["N"], shape["k"], shape["H"], shape["I"]
    B = args.batch
    layer_seed = 30 if args.config == "qwen30b" else 235

    # host weights (bf16 bits), stacked per matrix kind
    gate = np.empty((N, I, H), np.uint16)
    up = np.empty((N, I, H), np.uint16)
    down = np.empty((N, H, I), np.uint16)
    for e in range(N):
        gate[e], up[e], down[e] = synth.expert_weights_bf16(layer_seed, e, H, I)
    w_r = synth.router_weight(layer_seed, N, H)

    def to_dev(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    # pack each matrix into the tiled layout once; further layer copies are clones
    g0, u0, d0 = (moe.pack_weights(moe.MOE_W_BF16, to_dev(m).view(N * m.shape[1], m.shape[2]))[0]
                  .view(N, m.shape[1], m.shape[2]) for m in (gate, up, down))
    wr_dev = torch.from_numpy(w_r).to(dev)
    layers = []
    for c in range(args.copies):
        g, u, d = (g0, u0, d0) if c == 0 else (g0.clone(), u0.clone(), d0.clone())
        exps = [moe.ExpertTensors(moe.MOE_W_BF16, g[e], u[e], d[e]) for e in range(N)]
        layers.append(moe.MoELayer(H, I, N, k, wr_dev if c == 0 else wr_dev.clone(), exps, dev))
    xs_f32 = [synth.activations(b, B, H) for b in range(args.batches)]
    xs_bits = [synth.to_bf16_bits(x) for x in xs_f32]
    xs = [to_dev(x) for x in xs_bits]
    torch.cuda.synchronize()
    setup_s = time.time() - t_setup
    progress(f"setup done ({args.copies} layer copies)")

    W_e = 3 * H * I * 2                        # bf16 bytes per expert
    fixed_layer = N * H * 4 + B * H * 2 + B * H * 4
    fixed_ffn = B * H * 2 + B * H * 4

    def run_mode(mode, k0):
        # T per batch (identical for every layer copy: same weights), and the
        # routing's own counters: routed pairs, the cnt histogram over active
        # experts (bins 1, 2, 3-4, 5-8, 9-16, 17-32, 33-128 tokens), and the
        # tokens' baseline counts n_i (OEA)
        Ts, sum_cnt, hist, n_base = [], [], np.zeros(7, np.int64), []
        edges = np.array([1, 2, 3, 5, 9, 17, 33, 129])
        for b in range(args.batches):
            buf = layers[0].forward(xs[b], mode, k0, 1.0)
            Ts.append(int(buf.disp["T"].item()))
            cnt = buf.disp["cnt"].cpu().numpy()
            sum_cnt.append(int(cnt.sum()))
            hist += np.histogram(cnt[cnt > 0], bins=edges)[0]
            if mode == "oea":
                n_base.append(float(buf.route["n_base"].float().mean().item()))
        routing_counters = {"sum_cnt_mean": float(np.mean(sum_cnt)),
                            "cnt_hist_bins": ["1", "2", "3-4", "5-8", "9-16", "17-32", "33-128"],
                            "cnt_hist_per_batch": [round(float(h) / args.batches, 2) for h in hist],
                            "n_i_mean": round(float(np.mean(n_base)), 3) if n_base else None}
        stream = torch.cuda.current_stream()
        n_ev = args.steps
        evl = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
        ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
        ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]

        def step(i, timed):
            lay = layers[i % len(layers)]
            x = xs[i % len(xs)]
            buf = lay.buffers(B)
            if timed:
                evl[i].record(stream)
            # router GEMV + routing + dispatch: one launch
            moe.router_route_dispatch(x, lay.w_r, k, mode, k0, 1.0, True, buf.route, buf.disp, buf.logits,
                                      buf.extra["sync"])
            if timed:
                ev0[i].record(stream)
            lay.ffn(x, buf)
            if timed:
                ev1[i].record(stream)

        # whole-layer steps, no events in the stream
        for i in range(args.warmup):
            step(i, False)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(i, False)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        # the same steps again with HIP events around the expert FFN call
        for i in range(args.steps):
            step(i, True)
        torch.cuda.synchronize()
        ffn_ms = [ev0[i].elapsed_time(ev1[i]) for i in range(args.steps)]
        layer_ms = [evl[i].elapsed_time(ev1[i]) for i in range(args.steps)]
        # the same steps with the FFN call's three launches timed apart (events
        # recorded by the library between them, on the stream they run on)
        evp = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
        for i in range(args.steps):
            lay = layers[i % len(layers)]
            x = xs[i % len(xs)]
            buf = lay.buffers(B)
            moe.router_route_dispatch(x, lay.w_r, k, mode, k0, 1.0, True, buf.route, buf.disp, buf.logits,
                                      buf.extra["sync"])
            moe.expert_ffn_phase_events(lay.table, N, H, I, x, buf.route["idx"], buf.route["w"], buf.disp, buf.y,
                                        buf.ws, evp[i])
        torch.cuda.synchronize()
        phase_ms = [[evp[i][j].elapsed_time(evp[i][j + 1]) for i in range(args.steps)] for j in range(3)]
        # the same steps replayed from HIP graphs (one per layer copy and batch)
        graphs = {}
        for i in range(args.steps):
            key = (i % len(layers), i % len(xs))
            if key not in graphs:
                graphs[key] = layers[key[0]].capture(xs[key[1]], mode, k0, 1.0)
        for i in range(args.warmup):
            graphs[(i % len(layers), i % len(xs))].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            graphs[(i % len(layers), i % len(xs))].replay()
        torch.cuda.synchronize()
        graph_wall = time.perf_counter() - t0
        for i in range(args.steps):
            evl[i].record(stream)
            graphs[(i % len(layers), i % len(xs))].replay()
            ev1[i].record(stream)
        torch.cuda.synchronize()
        graph_ms = [evl[i].elapsed_time(ev1[i]) for i in range(args.steps)]
        del graphs
        # every layer copy in one graph (a decode step's MoE layers): one replay per step
        n_l = len(layers)
        g_all = moe.capture_layers([(layers[c], xs[c % len(xs)]) for c in range(n_l)], mode, k0, 1.0)
        n_rep = max(args.steps // n_l, 4)
        for i in range(2):
            g_all.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n_rep):
            g_all.replay()
        torch.cuda.synchronize()
        step_wall = time.perf_counter() - t0
        del g_all
        step_bytes = sum(Ts[c % len(Ts)] * W_e + fixed_layer for c in range(n_l))
        Tsteps = [Ts[i % len(Ts)] for i in range(args.steps)]
        layer_bytes = sum(t * W_e + fixed_layer for t in Tsteps)
        ffn_bytes = sum(t * W_e + fixed_ffn for t in Tsteps)
        ffn_s = sum(ffn_ms) / 1e3
        return dict(
            ms_per_step=wall / args.steps * 1e3,
            us_per_layer=wall / args.steps * 1e6,
            gbps=layer_bytes / wall / 1e9,
            T_mean=float(np.mean(Tsteps)),
            T_per_batch=Ts,
            routing_counters=routing_counters,
            ffn_us=ffn_s / args.steps * 1e6,
            ffn_us_p10=float(np.percentile(ffn_ms, 10) * 1e3),
            ffn_us_p50=float(np.percentile(ffn_ms, 50) * 1e3),
            ffn_us_p90=float(np.percentile(ffn_ms, 90) * 1e3),
            ffn_gbps=ffn_bytes / ffn_s / 1e9,
            ffn_bytes_per_launch=ffn_bytes / args.steps,
            layer_us_p10=float(np.percentile(layer_ms, 10) * 1e3),
            layer_us_p50=float(np.percentile(layer_ms, 50) * 1e3),
            layer_us_p90=float(np.percentile(layer_ms, 90) * 1e3),
            graph_us_per_layer=graph_wall / args.steps * 1e6,
            graph_us_p10=float(np.percentile(graph_ms, 10) * 1e3),
            graph_us_p50=float(np.percentile(graph_ms, 50) * 1e3),
            graph_us_p90=float(np.percentile(graph_ms, 90) * 1e3),
            graph_gbps=layer_bytes / graph_wall / 1e9,
            graph_step_us_per_layer=step_wall / (n_rep * n_l) * 1e6,
            graph_step_gbps=step_bytes * n_rep / step_wall / 1e9,
            phase_us=[float(np.mean(m) * 1e3) for m in phase_ms],
            phase_us_p50=[float(np.median(m) * 1e3) for m in phase_ms],
            phase_a_bytes_per_launch=float(np.mean([t * 2 * H * I * 2 for t in Tsteps])) + B * H * 2,
        )

    if args.only == "mixed":   # profiler runs of the mixed-residency layer alone (Qwen3-30B shape)
        print(json.dumps({"mixed_int4": mixed_int4(layers, wr_dev, N, k, H, I, gate, up, down)}), flush=True)
        return
    if args.only == "point":   # profiler runs of one batch-sweep point
        print(json.dumps({"point": point_run(layers, wr_dev, N, k, H, I, args)}), flush=True)
        return

    results = {}
    modes = [("oea", args.k0), ("topk", 0), ("oea", 5)]
    if args.only == "oea":
        modes = [("oea", args.k0)]
    elif args.only == "topk":
        modes = [("topk", 0)]
    for mode, k0 in modes:
        key = "oea_k0_%d" % k0 if mode == "oea" else "top%d" % k
        if key not in results:
            results[key] = run_mode(mode, k0)
            progress(f"{key}: FFN {results[key]['ffn_us']:.1f} us, layer p50 {results[key]['layer_us_p50']:.1f} us")
    head = results[list(results)[0]]

    # forced-T linearity: B tokens spread over T chosen experts (expert FFN only)
    sweep = None
    if not args.no_sweep and args.only is None:
        sweep = forced_t_sweep(layers, xs[0], B, N, k, W_e, fixed_ffn)
        progress("forced-T sweep done")

    ceiling = None
    if args.only is None:
        ceiling = read_ceiling()
        progress(f"read ceiling {ceiling['gbps']} GB/s")

    extended = None
    if not args.no_extended and args.only is None and args.config == "qwen30b":
        extended = {"small_batch_graphs": small_batch_graphs(layers, N, k, H)}
        progress("small-batch graphs done")
        extended["batch_sweep"] = batch_sweep(layers, wr_dev, N, k, H, I)
        progress("batch sweep done")
        extended["mixed_int4"] = mixed_int4(layers, wr_dev, N, k, H, I, gate, up, down)
        progress("mixed INT4 layer done")
        extended["dynamic_residency"] = dynamic_residency(wr_dev, N, k, H, I, gate, up, down)
        progress("dynamic residency done")
        del layers[:]
        torch.cuda.empty_cache()
        extended["qwen235b"] = qwen235b_lines()
        progress("Qwen3-235B-shaped layer done")

    cpu = None
    if not args.no_cpu_baseline and args.only is None:
        progress("CPU baseline (oracle) starting")
        cpu = cpu_baseline(args, N, k, H, I, B, gate, up, down, w_r, xs_bits, W_e)
        progress("CPU baseline done")

    out = {
        "metric": METRIC,
        "value": round(head["gbps"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.config} MoE layer decode, B={B}, N={N}, top-{k}, H={H}, I={I}, "
                               f"bf16 experts, routing {list(results)[0]}",
                   "batch": B, "layer_copies": args.copies, "batches": args.batches},
        "pct_peak": round(100 * head["gbps"] / HBM_PEAK_GBPS, 2),
        "results": {kk: {a: (round(b, 3) if isinstance(b, float) else b) for a, b in v.items()}
                    for kk, v in results.items()},
        "roofline": {
            "bound": "hbm",
            "kernel": "moe_expert_ffn (gate/up+SwiGLU, down+weight, combine)",
            "achieved": round(head["ffn_gbps"], 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(head["ffn_gbps"] / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic() if (args.config == "qwen30b" and B == 16 and args.k0 == 3) else None,
            "read_ceiling_gbps": None if ceiling is None else ceiling["gbps"],
            "frac_of_read_ceiling": None if ceiling is None else round(head["ffn_gbps"] / ceiling["gbps"], 4),
            "ffn_us_p10_p50_p90": [round(head["ffn_us_p10"], 2), round(head["ffn_us_p50"], 2),
                                   round(head["ffn_us_p90"], 2)],
        },
        "roofline_dominant_kernel": {
            "bound": "hbm",
            "kernel": "ffn_kernel<0> (phase A: gate/up + SwiGLU; the heaviest of the expert FFN's three launches)",
            "achieved": round(head["phase_a_bytes_per_launch"] / head["phase_us"][0] / 1e3, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(head["phase_a_bytes_per_launch"] / head["phase_us"][0] / 1e3 / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic("phase_a_") if (args.config == "qwen30b" and B == 16 and args.k0 == 3)
                       else None,
            "bytes_per_launch": round(head["phase_a_bytes_per_launch"]),
            "us_mean": round(head["phase_us"][0], 2),
            "us_p50": round(head["phase_us_p50"][0], 2),
            "phase_us_mean_a_b_combine": [round(v, 2) for v in head["phase_us"]],
        },
        "layer_us_p10_p50_p90": [round(head["layer_us_p10"], 2), round(head["layer_us_p50"], 2),
                                 round(head["layer_us_p90"], 2)],
        "read_ceiling": ceiling,
        "linearity": sweep,
        "extended": extended,
        "cpu_baseline": cpu,
        "setup_s": round(setup_s, 1),
    }
    print(json.dumps(out), flush=True)


def forced_t_sweep(layers, x, B, N, k, W_e, fixed_ffn, reps=40):
    """Latency of the expert FFN when B tokens are spread over exactly T experts
    (each token keeps k distinct experts of the chosen set); least-squares fit
    latency = b*T + c and its R^2 (page OEA section 3, Figure 1's linear fit)."""
    import numpy as np
    import torch

    import aware_expert_routing_amd as moe

    pts = []
    stream = torch.cuda.current_stream()
    for T in (8, 16, 24, 32, 48, 64, 80, 96, 112, 128):
        idx = np.empty((B, k), np.int32)
        for i in range(B):
            idx[i] = [(i * k + s) % T for s in range(k)] if T >= k else list(range(k))
        idx_d = torch.from_numpy(idx).to(layers[0].device)
        w_d = torch.full((B, k), 1.0 / k, device=layers[0].device)
        bufs = []
        for lay in layers:
            buf = lay.buffers(B)
            buf.route["idx"].copy_(idx_d)
            buf.route["w"].copy_(w_d)
            moe.dispatch(buf.route["idx"], N, buf.disp)
            bufs.append(buf)
        Tgot = int(bufs[0].disp["T"].item())
        e0 = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
        e1 = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
        for i in range(4):
            layers[i % len(layers)].ffn(x, bufs[i % len(layers)])
        for i in range(reps):
            lay = layers[i % len(layers)]
            e0[i].record(stream)
            lay.ffn(x, bufs[i % len(layers)])
            e1[i].record(stream)
        torch.cuda.synchronize()
        us = float(np.median([e0[i].elapsed_time(e1[i]) * 1e3 for i in range(reps)]))
        pts.append((Tgot, us, (Tgot * W_e + fixed_ffn) / us / 1e3))
    T = np.array([p[0] for p in pts], np.float64)
    y = np.array([p[1] for p in pts], np.float64)
    A = np.stack([T, np.ones_like(T)], 1)
    coef, *_ = np.linalg.lstsq(A, y, rcond=None)
    pred = A @ coef
    r2 = 1.0 - float(((y - pred) ** 2).sum() / ((y - y.mean()) ** 2).sum())
    return {"fit": "us = b*T + c", "b_us_per_expert": round(float(coef[0]), 4), "c_us": round(float(coef[1]), 3),
            "r2": round(r2, 6), "points": [{"T": int(t), "ffn_us": round(u, 2), "gbps": round(g, 1)} for t, u, g in pts]}


def _fit(T, y, extra=None):
    """Least squares y = b*T (+ a*extra) + c; returns coefficients and R^2."""
    import numpy as np
    cols = [np.asarray(T, np.float64)] + ([np.asarray(extra, np.float64)] if extra is not None else [])
    A = np.stack(cols + [np.ones(len(T))], 1)
    y = np.asarray(y, np.float64)
    coef, *_ = np.linalg.lstsq(A, y, rcond=None)
    pred = A @ coef
    r2 = 1.0 - float(((y - pred) ** 2).sum() / ((y - y.mean()) ** 2).sum())
    return [round(float(c), 4) for c in coef], round(r2, 5)


def _time_steps(step, n, warm=3):
    import torch
    for i in range(warm):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n):
        step(i)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / n * 1e6


def _graph_us(call, reps=16, replays=20):
    """GPU time of one call: `reps` calls captured in one HIP graph, replayed
    `replays` times (the graph's own launch cost is spread over the reps)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            call()
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(replays):
        g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / (reps * replays) * 1e6


def batch_sweep(layers, w_r, N, k, H, I, batches=5, steps=30):
    """Routing + dispatch + expert FFN latency and T over B = 1..128 for
    vanilla top-8, simplified OEA (k0 = 3, 5) and full OEA (k0 in {3, 5},
    p in {0.5, 0.7, 0.9}), with router logits plus a Zipf(1.1) expert bias
    and with the uniform control.  The router GEMV runs once per batch
    outside the timed steps (the bias is added to its output); its own cost
    is reported per B.  Fits latency = b*T + c and b*T + a*sum(cnt) + c
    (page OEA section 4, Eq. 2) over all points of each routing family."""
    import numpy as np
    import torch

    import aware_expert_routing_amd as moe
    import synth

    dev = layers[0].device
    W_e = 3 * H * I * 2
    routings = [("topk", 0, 1.0)] + [("oea", k0, p) for k0 in (3, 5) for p in (1.0, 0.5, 0.7, 0.9)]
    points, router_us = [], {}
    for B in (1, 2, 4, 8, 16, 32, 64, 128):
        xs = [torch.from_numpy(synth.to_bf16_bits(synth.activations(100 + b, B, H)).view(np.int16)).to(dev)
              .view(torch.bfloat16) for b in range(batches)]
        base = [moe.router_logits(x, w_r) for x in xs]
        router_us[B] = round(_graph_us(lambda: moe.router_logits(xs[0], w_r, layers[0].buffers(B).logits)), 2)
        for zipf in (1.1, 0.0):
            beta = torch.from_numpy(synth.zipf_bias(N, zipf)).to(dev)
            logits = [l + beta[None, :] for l in base]
            for mode, k0, p in routings:
                Ts, sc = [], []
                for b in range(batches):
                    buf = layers[0].buffers(B)
                    layers[0].route(logits[b], mode, k0, p, buf)
                    Ts.append(int(buf.disp["T"].item()))
                    sc.append(int(buf.disp["offsets"][N].item()))

                def step(i):
                    lay = layers[i % len(layers)]
                    buf = lay.buffers(B)
                    lay.route(logits[i % batches], mode, k0, p, buf)
                    lay.ffn(xs[i % batches], buf)
                us = _time_steps(step, steps)
                T = float(np.mean(Ts))
                points.append(dict(B=B, routing=mode if mode == "topk" else f"oea_k0_{k0}_p{p}", zipf=zipf,
                                   T=round(T, 2), sum_cnt=round(float(np.mean(sc)), 1), us=round(us, 2),
                                   gbps=round(T * W_e / us / 1e3, 1)))
    fits = {}
    for fam in ("topk", "oea"):
        sel = [q for q in points if q["routing"].startswith(fam)]
        c1, r1 = _fit([q["T"] for q in sel], [q["us"] for q in sel])
        c2, r2 = _fit([q["T"] for q in sel], [q["us"] for q in sel], [q["sum_cnt"] for q in sel])
        fits[fam] = {"us = b*T + c": {"b": c1[0], "c": c1[1], "r2": r1},
                     "us = b*T + a*sum_cnt + c": {"b": c2[0], "a": c2[1], "c": c2[2], "r2": r2}}
    return {"what": "route+dispatch+expert FFN per step, logits given (router GEMV timed apart, GPU time from a "
                    "graph of 16 calls)",
            "router_us": router_us, "fits": fits, "points": points}


def mixed_int4(layers, w_r, N, k, H, I, gate, up, down, B=32, warm=64, hot=32, copies=8, steps=60):
    """Qwen3-30B shape with a handle table of the `hot` hottest experts in
    bf16 and the rest in INT4 (group 128), the hot set taken from an EMA of
    vanilla top-8 routing counts (alpha 0.9) over `warm` Zipf-biased batches
    (page DynaExq sections 2.5 / 3.2).  B = 32; vanilla top-8 vs OEA k0=5."""
    import numpy as np
    import torch

    import aware_expert_routing_amd as moe
    import synth

    dev = layers[0].device
    beta = torch.from_numpy(synth.zipf_bias(N, 1.1)).to(dev)
    xs_warm = [torch.from_numpy(synth.to_bf16_bits(synth.activations(200 + b, B, H)).view(np.int16)).to(dev)
               .view(torch.bfloat16) for b in range(warm)]
    hot_set = set(moe.ema_hot_set(xs_warm, w_r, beta, k, hot, 0.9))

    def dev_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    experts = []
    for e in range(N):
        mats = [dev_bf16(gate[e]), dev_bf16(up[e]), dev_bf16(down[e])]
        if e in hot_set:
            experts.append(moe.ExpertTensors.pack(moe.MOE_W_BF16, *mats))
        else:
            q = [moe.quantize_int4_g128(m) for m in mats]
            experts.append(moe.ExpertTensors.pack(moe.MOE_W_INT4_G128, q[0][0], q[1][0], q[2][0],
                                                  q[0][1], q[1][1], q[2][1]))
    mlayers = [moe.MoELayer(H, I, N, k, w_r, experts, dev)]
    for c in range(1, copies):
        ex = [moe.ExpertTensors(t.fmt, t.gate.clone(), t.up.clone(), t.down.clone(),
                                None if t.s_gate is None else t.s_gate.clone(),
                                None if t.s_up is None else t.s_up.clone(),
                                None if t.s_down is None else t.s_down.clone()) for t in experts]
        mlayers.append(moe.MoELayer(H, I, N, k, w_r, ex, dev))
    bf16_bytes = 3 * H * I * 2
    int4_bytes = 3 * (H * I // 2 + H * I // 128 * 2)
    xs = [torch.from_numpy(synth.to_bf16_bits(synth.activations(300 + b, B, H)).view(np.int16)).to(dev)
          .view(torch.bfloat16) for b in range(10)]
    logits = [moe.router_logits(x, w_r) + beta[None, :] for x in xs]
    out = {"B": B, "hot_bf16": hot, "cold_int4": N - hot,
           "layer_bytes": hot * bf16_bytes + (N - hot) * int4_bytes}
    for mode, k0 in (("topk", 0), ("oea", 5)):
        Ts, byts = [], []
        for b in range(10):
            buf = mlayers[0].buffers(B)
            mlayers[0].route(logits[b], mode, k0, 1.0, buf)
            act = buf.disp["active"].cpu().numpy()
            T = int(buf.disp["T"].item())
            Ts.append(T)
            byts.append(sum(bf16_bytes if int(e) in hot_set else int4_bytes for e in act[:T]))

        def step(i):
            lay = mlayers[i % copies]
            buf = lay.buffers(B)
            lay.route(logits[i % 10], mode, k0, 1.0, buf)
            lay.ffn(xs[i % 10], buf)
        us = _time_steps(step, steps)
        key = "top8" if mode == "topk" else "oea_k0_5"
        out[key] = {"T": round(float(np.mean(Ts)), 2), "us": round(us, 2),
                    "weight_bytes": round(float(np.mean(byts))),
                    "gbps": round(float(np.mean(byts)) / us / 1e3, 1)}
    del mlayers
    return out


def dynamic_residency(w_r, N, k, H, I, gate, up, down, B=32, n_hi=32, alpha=0.9, margin=0.5, period=8,
                      phase_steps=48):
    """Online residency on the Qwen3-30B shape (page DynaExq, 2.2-2.5 / 3.2-3.5):
    every expert resident in INT4, bf16 versions in pinned host memory, 32
    high-precision blocks.  Vanilla top-8 routing with a Zipf(1.1) bias whose
    expert order changes every `phase_steps` steps; a policy update every
    `period` steps; copies run on the migration stream while the layer runs.
    Reports the layer's compute-stream time per step with and without copies
    in flight, and the promotions' host-to-device rate."""
    import numpy as np
    import torch

    import aware_expert_routing_amd as moe
    import synth

    dev = w_r.device

    def dev_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    lo, hi_host = [], []
    for e in range(N):
        mats = [dev_bf16(gate[e]), dev_bf16(up[e]), dev_bf16(down[e])]
        q = [moe.quantize_int4_g128(m) for m in mats]
        lo.append(moe.ExpertTensors.pack(moe.MOE_W_INT4_G128, q[0][0], q[1][0], q[2][0], q[0][1], q[1][1],
                                         q[2][1]))
        hi_host.append(moe.pinned_hi_version(moe.ExpertTensors.pack(moe.MOE_W_BF16, *mats)))
    layer = moe.MoELayer(H, I, N, k, w_r, lo, dev)
    torch.cuda.synchronize()
    res = moe.Residency(layer, lo, hi_host, n_hi, alpha=alpha, margin=margin)
    xs = [dev_bf16(synth.to_bf16_bits(synth.activations(700 + b, B, H))) for b in range(10)]
    base = [moe.router_logits(x, w_r) for x in xs]
    biases = [torch.from_numpy(synth.zipf_bias(N, 1.1, seed=40 + ph)).to(dev) for ph in range(3)]
    quiet, busy = [], []
    t_update, settle = None, []
    try:
        for i in range(3 * phase_steps):
            logits = base[i % 10] + biases[i // phase_steps][None, :]
            inflight = any(s in (moe.MOE_RES_PROMOTING, moe.MOE_RES_EVICTING) for s in res.states())
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            buf = layer.forward(xs[i % 10], "topk", logits=logits)
            e1.record()
            force = i % period == period - 1
            res.step(buf.disp["cnt"], force=force)
            e1.synchronize()
            (busy if inflight else quiet).append(e0.elapsed_time(e1) * 1e3)
            now = time.perf_counter()
            if force:
                t_update = (now, res.stats()["bytes_h2d"])
            elif t_update is not None and not any(
                    s in (moe.MOE_RES_PROMOTING, moe.MOE_RES_EVICTING) for s in res.states()) \
                    and res.pending() == 0 and res.stats()["decisions"] == res.stats()["updates"]:
                moved = res.stats()["bytes_h2d"] - t_update[1]
                if moved:
                    settle.append((moved, now - t_update[0]))
                t_update = None
        st = res.stats()
    finally:
        res.close()
        del layer
    moved = sum(m for m, _ in settle)
    span = sum(t for _, t in settle)
    return {"B": B, "n_hi": n_hi, "alpha": alpha, "margin": margin, "update_every_steps": period,
            "steps": 3 * phase_steps, "stats": st,
            "layer_us_quiet": round(float(np.median(quiet)), 2) if quiet else None,
            "layer_us_copies_in_flight": round(float(np.median(busy)), 2) if busy else None,
            "steps_with_copies_in_flight": len(busy),
            "promotion_h2d_gbps": round(moved / span / 1e9, 2) if span else None,
            "note": "layer time from events on the compute stream (router GEMV + routing + FFN); "
                    "H2D rate = bytes promoted per update / wall time from the update to settled states"}


def qwen235b_lines(copies=2, steps=30):
    """Qwen3-235B-A22B-shaped layer (H=4096, I=1536, 37.7 MB per bf16 expert,
    4.83 GB per layer) on one GPU; seeded N(0, 0.02) weights drawn on the
    device.  B in {16, 32, 64}; vanilla top-8 vs OEA k0=5; router logits from
    the layer's own router; whole-layer steps."""
    import numpy as np
    import torch

    import aware_expert_routing_amd as moe
    import synth

    from concurrent.futures import ThreadPoolExecutor

    dev = torch.device("cuda:0")
    s = synth.SHAPES["qwen235b"]
    N, k, H, I = s["N"], s["k"], s["H"], s["I"]
    w_r = torch.from_numpy(synth.router_weight(235, N, H)).to(dev)
    packed = [torch.empty(N, rows, cols, device=dev, dtype=torch.bfloat16) for rows, cols in ((I, H), (I, H), (H, I))]
    with ThreadPoolExecutor(8) as ex:   # the seeded host generator of the parity tests (layer seed 235)
        for e, mats in enumerate(ex.map(lambda e: synth.expert_weights_bf16(235, e, H, I), range(N))):
            for m, dst in zip(mats, packed):
                src = torch.from_numpy(m.view(np.int16)).to(dev).view(torch.bfloat16)
                moe.pack_weights(moe.MOE_W_BF16, src, dst=dst[e])
    layers = []
    for c in range(copies):
        mats = packed if c == 0 else [t.clone() for t in packed]
        layers.append(moe.MoELayer(H, I, N, k, w_r, [moe.ExpertTensors(moe.MOE_W_BF16, mats[0][e], mats[1][e],
                                                                       mats[2][e]) for e in range(N)], dev))
    W_e = 3 * H * I * 2
    out = {"H": H, "I": I, "expert_bytes": W_e, "points": []}
    for B in (16, 32, 64):
        xs = [torch.from_numpy(synth.to_bf16_bits(synth.activations(400 + b, B, H)).view(np.int16)).to(dev)
              .view(torch.bfloat16) for b in range(4)]
        for mode, k0 in (("topk", 0), ("oea", 5)):
            Ts = []
            for b in range(4):
                Ts.append(int(layers[0].forward(xs[b], mode, k0, 1.0).disp["T"].item()))

            def step(i):
                layers[i % copies].forward(xs[i % 4], mode, k0, 1.0)
            us = _time_steps(step, steps)
            T = float(np.mean(Ts))
            out["points"].append(dict(B=B, routing="top8" if mode == "topk" else "oea_k0_5", T=round(T, 2),
                                      us=round(us, 2), gbps=round((T * W_e + N * H * 4) / us / 1e3, 1)))
    del layers
    torch.cuda.empty_cache()
    return out


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(args, N, k, H, I, B, gate, up, down, w_r, xs_bits, W_e, reps=5):
    """The oracle (plain C, fp64; OpenMP across routed pairs and rows, the
    combine sequential, so the result does not depend on the thread count)
    on whole layers (router logits, routing, expert FFN): the median of
    `reps` calls at B = 16 (the benchmark's first batch), 1 and 128, for OEA
    k0 = args.k0 and vanilla top-k, with every host thread the oracle is
    given, and at the headline point (B = 16, OEA) on one thread."""
    import numpy as np

    import oracle
    import synth

    experts = [dict(fmt=oracle.FMT_BF16, gate=gate[e], up=up[e], down=down[e]) for e in range(N)]
    wr64 = w_r.astype(np.float64)

    def layer_call(x64, mode, k0):
        logits = oracle.router_logits(x64, wr64).astype(np.float32)
        r = oracle.route(logits, k, oea=(mode == "oea"), k0=k0, p=1.0)
        oracle.expert_ffn(experts, H, I, x64, r["idx"], r["w"])
        return r["T"]

    def timed(x64, mode, k0, n):
        ts, T = [], 0
        for _ in range(n):
            t0 = time.perf_counter()
            T = layer_call(x64, mode, k0)
            ts.append(time.perf_counter() - t0)
        return float(np.median(ts)), T

    threads = oracle.get_threads()
    t_all = time.perf_counter()
    points = []
    for Bp in (B, 1, 128):
        bits = xs_bits[0] if Bp == B else synth.to_bf16_bits(synth.activations(500, Bp, H))
        x64 = synth.bf16_bits_to_f32(bits).astype(np.float64)
        for mode, k0 in (("oea", args.k0), ("topk", 0)):
            med, T = timed(x64, mode, k0, reps)
            nbytes = T * W_e + N * H * 4 + Bp * H * 2 + Bp * H * 4
            points.append({"B": Bp, "routing": f"oea_k0_{k0}" if mode == "oea" else f"top{k}", "T": T,
                           "threads": threads, "median_s": round(med, 4), "gbps": round(nbytes / med / 1e9, 4)})
    head = points[0]
    x64 = synth.bf16_bits_to_f32(xs_bits[0]).astype(np.float64)
    try:
        oracle.set_threads(1)
        med1, T1 = timed(x64, "oea", args.k0, reps)
    finally:
        oracle.set_threads(threads)
    nbytes = T1 * W_e + N * H * 4 + B * H * 2 + B * H * 4
    single = {"B": B, "routing": head["routing"], "T": T1, "threads": 1, "median_s": round(med1, 4),
              "gbps": round(nbytes / med1 / 1e9, 4)}
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    return {"value": head["gbps"], "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"median of {reps} whole-layer oracle calls (router logits, routing, expert FFN) per point: "
                      f"B={B} (the benchmark's first batch), 1 and 128, OEA k0={args.k0} and top-{k}, "
                      f"{threads} threads (OpenMP, fp64); value = B={B} OEA k0={args.k0}; plus that point on one "
                      f"thread; {time.perf_counter() - t_all:.1f} s in all",
            "cpu_model": cpu_model(), "nproc": os.cpu_count(), "affinity_cpus": affinity,
            "us_per_layer": round(head["median_s"] * 1e6, 1), "points": points, "single_thread": single}


def read_ceiling(gib=4, reps=10, shapes=(4, 8, 16, 32)):
    """HBM read-stream ceiling: moe_stream_read (each wave a contiguous run of
    kilobytes, 16-byte non-temporal loads, one pass) over a 4 GiB buffer, for
    several waves per compute unit; the median over `reps` timed passes of
    the best shape."""
    import numpy as np
    import torch

    import aware_expert_routing_amd as moe

    nbytes = gib << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    buf.fill_(0x5A)
    out = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream()
    by_shape = {}
    for wpc in shapes:
        for _ in range(2):
            moe.stream_read(buf, out, wpc)
        e0 = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
        e1 = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
        for i in range(reps):
            e0[i].record(stream)
            moe.stream_read(buf, out, wpc)
            e1[i].record(stream)
        torch.cuda.synchronize()
        by_shape[wpc] = float(np.median([e0[i].elapsed_time(e1[i]) for i in range(reps)]))
    del buf
    torch.cuda.empty_cache()
    best = min(by_shape, key=by_shape.get)
    ms = by_shape[best]
    return {"kernel": "moe_stream_read", "bytes": nbytes, "waves_per_cu": best, "us": round(ms * 1e3, 2),
            "gbps": round(nbytes / ms / 1e6, 1), "frac_of_peak": round(nbytes / ms / 1e6 / HBM_PEAK_GBPS, 4),
            "gbps_by_waves_per_cu": {str(w): round(nbytes / t / 1e6, 1) for w, t in by_shape.items()}}


def small_batch_graphs(layers, N, k, H, steps=60):
    """Whole-layer latency (router GEMV + routing + dispatch + expert FFN) at
    B = 1, 2, 4, 8 (page OEA section 7: graph replay of small decode
    batches), OEA k0 = 3 and vanilla top-8; medians of per-step HIP events:
    eager launches against one captured HIP graph per layer copy, and the 8
    layer copies as one decode step, eager against one graph of all 8
    (per layer), the graph also from cold caches (a 1 GB buffer written and
    read before each step, outside its events).  host_us: the host's time per
    layer call, eager forward against the 8-layer graph's replay, without
    synchronisation."""
    import numpy as np
    import torch

    import aware_expert_routing_amd as moe
    import synth

    dev = layers[0].device
    stream = torch.cuda.current_stream()
    # written and read before each cold step (outside its events): 1 GB, more
    # than the L2s and the 256 MB MALL hold, so no weights survive in a cache
    flush = torch.zeros(1 << 28, device=dev, dtype=torch.float32)
    out = []
    for B in (1, 2, 4, 8):
        xs = [torch.from_numpy(synth.to_bf16_bits(synth.activations(600 + c, B, H)).view(np.int16)).to(dev)
              .view(torch.bfloat16) for c in range(len(layers))]
        for mode, k0 in (("oea", 3), ("topk", 0)):
            e0 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
            e1 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]

            def eager(i, timed=True):
                c = i % len(layers)
                if timed:
                    e0[i].record(stream)
                layers[c].forward(xs[c], mode, k0, 1.0)
                if timed:
                    e1[i].record(stream)
            for i in range(8):
                eager(i, False)
            for i in range(steps):
                eager(i)
            torch.cuda.synchronize()
            eager_us = float(np.median([e0[i].elapsed_time(e1[i]) for i in range(steps)])) * 1e3
            graphs = [layers[c].capture(xs[c], mode, k0, 1.0) for c in range(len(layers))]
            for i in range(8):
                graphs[i % len(graphs)].replay()
            for i in range(steps):
                e0[i].record(stream)
                graphs[i % len(graphs)].replay()
                e1[i].record(stream)
            torch.cuda.synchronize()
            graph_us = float(np.median([e0[i].elapsed_time(e1[i]) for i in range(steps)])) * 1e3
            del graphs
            # the 8 copies as one decode step: eager, then one graph of all of them
            n_l = len(layers)
            reps = max(steps // 4, 8)
            for i in range(reps):
                e0[i].record(stream)
                for c in range(n_l):
                    layers[c].forward(xs[c], mode, k0, 1.0)
                e1[i].record(stream)
            torch.cuda.synchronize()
            eager_step = float(np.median([e0[i].elapsed_time(e1[i]) for i in range(reps)])) * 1e3
            g_all = moe.capture_layers(list(zip(layers, xs)), mode, k0, 1.0)
            for i in range(2):
                g_all.replay()
            for i in range(reps):
                e0[i].record(stream)
                g_all.replay()
                e1[i].record(stream)
            torch.cuda.synchronize()
            graph_step = float(np.median([e0[i].elapsed_time(e1[i]) for i in range(reps)])) * 1e3
            # the same replays from cold caches (the step's expert weights at
            # B = 1, OEA k0 = 3 -- 8 x 3 experts, 226 MB -- would fit the MALL)
            for i in range(reps):
                flush.add_(1.0)
                e0[i].record(stream)
                g_all.replay()
                e1[i].record(stream)
            torch.cuda.synchronize()
            graph_step_cold = float(np.median([e0[i].elapsed_time(e1[i]) for i in range(reps)])) * 1e3
            t0 = time.perf_counter()
            for i in range(reps):
                g_all.replay()
            host_graph = (time.perf_counter() - t0) / (reps * n_l) * 1e6
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(reps):
                for c in range(n_l):
                    layers[c].forward(xs[c], mode, k0, 1.0)
            host_eager = (time.perf_counter() - t0) / (reps * n_l) * 1e6
            torch.cuda.synchronize()
            del g_all
            T = int(layers[0].forward(xs[0], mode, k0, 1.0).disp["T"].item())
            out.append({"B": B, "routing": f"oea_k0_{k0}" if mode == "oea" else f"top{k}", "T_first_copy": T,
                        "eager_us": round(eager_us, 2), "graph_us": round(graph_us, 2),
                        "step_of_%d_layers" % n_l: {"eager_us_per_layer": round(eager_step / n_l, 2),
                                                    "graph_us_per_layer": round(graph_step / n_l, 2),
                                                    "graph_us_per_layer_cold": round(graph_step_cold / n_l, 2),
                                                    "host_us_per_layer_eager": round(host_eager, 1),
                                                    "host_us_per_layer_graph": round(host_graph, 1)}})
    return out


def point_run(layers, w_r, N, k, H, I, args):
    """One batch-sweep point alone (routing + dispatch + expert FFN per step,
    router logits plus a Zipf bias given), for counter runs."""
    import numpy as np
    import torch

    import aware_expert_routing_amd as moe
    import synth

    dev = layers[0].device
    B, mode, k0 = args.batch, args.routing, (args.k0 if args.routing == "oea" else 0)
    beta = torch.from_numpy(synth.zipf_bias(N, args.zipf)).to(dev)
    xs = [torch.from_numpy(synth.to_bf16_bits(synth.activations(100 + b, B, H)).view(np.int16)).to(dev)
          .view(torch.bfloat16) for b in range(5)]
    logits = [moe.router_logits(x, w_r) + beta[None, :] for x in xs]
    Ts, sc = [], []
    for b in range(5):
        buf = layers[0].buffers(B)
        layers[0].route(logits[b], mode, k0, 1.0, buf)
        Ts.append(int(buf.disp["T"].item()))
        sc.append(int(buf.disp["offsets"][N].item()))

    def step(i):
        lay = layers[i % len(layers)]
        buf = lay.buffers(B)
        lay.route(logits[i % 5], mode, k0, 1.0, buf)
        lay.ffn(xs[i % 5], buf)
    us = _time_steps(step, args.steps, warm=args.warmup)
    W_e = 3 * H * I * 2
    T = float(np.mean(Ts))
    return {"B": B, "routing": mode, "k0": k0, "zipf": args.zipf, "T": T, "sum_cnt": float(np.mean(sc)),
            "steps": args.steps, "us": round(us, 2), "gbps": round(T * W_e / us / 1e3, 1)}


if __name__ == "__main__":
    main()
