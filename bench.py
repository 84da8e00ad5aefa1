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
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--only", choices=["oea", "topk"], default=None,
                    help="time only this routing (for profiler runs)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run 20 plain device copies of MIB MiB (the "
                         "reference kernel for scaling HBM byte counters) and exit")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "expert_ffn_traffic_qwen30b_b16_oea3.txt")
FFN_SOURCES = [os.path.join(ROOT, "aware_expert_routing_amd", "csrc", f) for f in ("ffn.hip", "pack.hip")]


def sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in FFN_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per expert-FFN call from the committed counter summary, or
    None when it is missing or was taken on different kernel sources."""
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
        return int(float(kv["fetch_bytes_per_call"]) + float(kv["write_bytes_per_call"]))
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
        print(json.dumps({"error": "this build runs on exactly one GPU; --gpus must be 1",
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

    W_e = 3 * H * I * 2                        # bf16 bytes per expert
    fixed_layer = N * H * 4 + B * H * 2 + B * H * 4
    fixed_ffn = B * H * 2 + B * H * 4

    def run_mode(mode, k0):
        # T per batch (identical for every layer copy: same weights)
        Ts = []
        for b in range(args.batches):
            buf = layers[0].forward(xs[b], mode, k0, 1.0)
            Ts.append(int(buf.disp["T"].item()))
        stream = torch.cuda.current_stream()
        n_ev = args.steps
        ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
        ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]

        def step(i, timed):
            lay = layers[i % len(layers)]
            x = xs[i % len(xs)]
            buf = lay.buffers(B)
            moe.router_logits(x, lay.w_r, buf.logits)
            lay.route(buf.logits, mode, k0, 1.0, buf)
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
            ffn_us=ffn_s / args.steps * 1e6,
            ffn_us_p10=float(np.percentile(ffn_ms, 10) * 1e3),
            ffn_us_p90=float(np.percentile(ffn_ms, 90) * 1e3),
            ffn_gbps=ffn_bytes / ffn_s / 1e9,
            ffn_bytes_per_launch=ffn_bytes / args.steps,
        )

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
    head = results[list(results)[0]]

    # forced-T linearity: B tokens spread over T chosen experts (expert FFN only)
    sweep = None
    if not args.no_sweep and args.only is None:
        sweep = forced_t_sweep(layers, xs[0], B, N, k, W_e, fixed_ffn)

    cpu = None
    if not args.no_cpu_baseline and args.only is None:
        cpu = cpu_baseline(args, N, k, H, I, B, gate, up, down, w_r, xs_bits, W_e, fixed_layer)

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
        },
        "linearity": sweep,
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


def cpu_baseline(args, N, k, H, I, B, gate, up, down, w_r, xs_bits, W_e, fixed_layer):
    """The oracle (plain C, one thread, fp64) on a bounded sample of the same
    workload: whole layers (router logits, OEA routing, expert FFN) on as many
    of the benchmark's batches as fit in about --cpu-seconds."""
    import numpy as np

    import oracle
    import synth

    experts = [dict(fmt=oracle.FMT_BF16, gate=gate[e], up=up[e], down=down[e]) for e in range(N)]
    wr64 = w_r.astype(np.float64)
    done, bytes_done, t0 = 0, 0, time.perf_counter()
    while True:
        x = synth.bf16_bits_to_f32(xs_bits[done % len(xs_bits)]).astype(np.float64)
        logits = oracle.router_logits(x, wr64).astype(np.float32)
        r = oracle.route(logits, k, oea=True, k0=args.k0, p=1.0)
        oracle.expert_ffn(experts, H, I, x, r["idx"], r["w"])
        bytes_done += r["T"] * W_e + fixed_layer
        done += 1
        el = time.perf_counter() - t0
        if el >= args.cpu_seconds or done >= 50:
            break
    return {"value": round(bytes_done / el / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} whole-layer calls (B={B}, OEA k0={args.k0}) of the benchmark's batches, "
                      f"{el:.1f} s, single-threaded C oracle (fp64)",
            "us_per_layer": round(el / done * 1e6, 1)}


if __name__ == "__main__":
    main()
