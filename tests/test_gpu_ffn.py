"""GPU parity of the expert FFN (SwiGLU + weighted combine) and of the whole
decode layer against the CPU oracle.

Bar: max|y - y_ref| <= 1e-2 * rms(y_ref) for bf16 experts (fp32 accumulate),
<= 2e-2 * rms(y_ref) for INT4 group-128 experts, and a tighter 1e-4 for fp32
experts (fp32 products and sums over at most a few thousand terms).
Page "Opportunistic Expert Activation (OEA) - L2", section 4 (Eq. 2, check 4);
page "DynaExq", section 2.2 / 3.2 (handles, INT4 low-precision versions).
"""
import numpy as np
import pytest
import torch

import aware_expert_routing_amd as moe
import oracle
import synth
from gpu_util import DEV, bf16_dev, build_layer, max_err_over_rms, routing_order_is_robust

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 1e-2, "int4": 2e-2}


def _run_and_check(layer, host, x_np, x_dev, logits, mode, k0, p, tol, tokens=None):
    buf = layer.forward(x_dev, mode, k0, p, logits=torch.from_numpy(logits).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.route(logits, layer.k, oea=(mode == "oea"), k0=k0, p=p)
    assert np.array_equal(buf.route["idx"].cpu().numpy(), ref["idx"])
    rows = np.arange(x_np.shape[0]) if tokens is None else np.asarray(tokens)
    yref = oracle.expert_ffn(host, layer.H, layer.I, x_np[rows], ref["idx"][rows], ref["w"][rows])
    err, rms = max_err_over_rms(buf.y[torch.from_numpy(rows).to(DEV)], yref)
    assert err <= tol * rms, (err, rms, err / rms)
    return buf, err / rms


def _x(seed, B, H, dtype):
    x = synth.activations(seed, B, H)
    if dtype == "bf16":
        xb = synth.to_bf16_bits(x)
        return synth.bf16_bits_to_f32(xb), bf16_dev(xb)
    return x, torch.from_numpy(x).to(DEV)


def test_tiny_fp32_layer_vanilla_and_oea():
    N, k, H, I, B = 16, 4, 256, 128, 4
    layer, host = build_layer(N, k, H, I, 1, fmt="f32", with_router=False)
    x, xd = _x(1, B, H, "f32")
    for scale in (1.0, 8.0):
        logits = synth.logits(1, B, N, scale)
        _run_and_check(layer, host, x, xd, logits, "topk", 0, 1.0, TOL["f32"])
        _run_and_check(layer, host, x, xd, logits, "oea", 2, 0.7, TOL["f32"])


@pytest.mark.parametrize("N,k,H,I,B,mode,k0,p", [
    (16, 4, 544, 224, 24, "topk", 0, 1.0),    # odd tile counts; last phase-B item ragged
    (16, 4, 544, 224, 24, "oea", 2, 0.7),
    (8, 4, 256, 128, 64, "topk", 0, 1.0),     # > 32 tokens per expert: several passes
    (32, 16, 384, 288, 9, "topk", 0, 1.0),    # k = 16
    (128, 8, 256, 128, 128, "oea", 3, 1.0),   # B = 128
    (128, 8, 256, 128, 1, "oea", 3, 1.0),     # B = 1
    (12, 3, 1024, 640, 5, "oea", 1, 0.9),
])
def test_bf16_ffn_shapes(N, k, H, I, B, mode, k0, p):
    layer, host = build_layer(N, k, H, I, 2, fmt="bf16", with_router=False)
    x, xd = _x(2, B, H, "bf16")
    logits = synth.logits(2, B, N, 4.0)
    _run_and_check(layer, host, x, xd, logits, mode, k0, p, TOL["bf16"])


@pytest.mark.parametrize("fmt", ["bf16", "f32"])
def test_experts_with_two_column_tiles(fmt):
    # B=40 tokens over 4 experts, top-2: every active expert carries more than
    # 16 tokens, so both phases use two column tiles and phase B uses items of
    # 4 row blocks; H = 544 gives 34 row blocks, so the last phase-B item has
    # two clamped row blocks; B=80 adds a second token pass for some experts.
    for B, seed in ((40, 11), (80, 12)):
        N, k, H, I = 4, 2, 544, 224
        layer, host = build_layer(N, k, H, I, seed, fmt=fmt, with_router=False)
        x, xd = _x(seed, B, H, "bf16" if fmt == "bf16" else "f32")
        logits = synth.logits(seed, B, N, 1.0)
        buf, _ = _run_and_check(layer, host, x, xd, logits, "topk", 0, 1.0, TOL[fmt])
        assert buf.disp["cnt"].cpu().numpy().max() > 16


def test_fp32_activations_with_bf16_experts():
    N, k, H, I, B = 16, 4, 256, 128, 8
    layer, host = build_layer(N, k, H, I, 3, fmt="bf16", with_router=False)
    x = synth.activations(3, B, H)
    # the library rounds fp32 activations to bf16 for bf16 experts; the oracle sees exact x
    logits = synth.logits(3, B, N)
    _run_and_check(layer, host, x, torch.from_numpy(x).to(DEV), logits, "topk", 0, 1.0, TOL["bf16"])


@pytest.mark.parametrize("int4", ["all", "mixed"])
def test_int4_and_mixed_experts(int4):
    N, k, H, I, B = 16, 4, 512, 256, 32
    which = range(N) if int4 == "all" else range(4, N)       # 4 hot bf16, 12 cold INT4
    layer, host = build_layer(N, k, H, I, 4, fmt="bf16", int4_experts=which, with_router=False)
    # the GPU quantiser's INT4 bytes equal the oracle's, bit for bit (before packing)
    for e in which:
        q = layer.rowmajor_int4[e]
        for name in ("gate", "up", "down"):
            assert np.array_equal(q[name].cpu().numpy(), host[e][name])
            assert np.array_equal(q["s_" + name].cpu().numpy().view(np.uint16), host[e]["s_" + name])
    x, xd = _x(4, B, H, "bf16")
    logits = (synth.logits(4, B, N, 1.0) + synth.zipf_bias(N, 1.1)[None, :]).astype(np.float32)
    buf, _ = _run_and_check(layer, host, x, xd, logits, "topk", 0, 1.0, TOL["int4"])
    if int4 == "all":   # Zipf-hot INT4 experts take more than one pass of 16 tokens
        assert buf.disp["cnt"].cpu().numpy().max() > 16
    _run_and_check(layer, host, x, xd, logits, "oea", 2, 1.0, TOL["int4"])


def test_int4_experts_with_fp32_activations():
    # fp32 x meets INT4 tiles as bf16 hi + lo pairs (one activation stage,
    # deeper weight ring); h then enters the down projection in bf16
    N, k, H, I, B = 8, 2, 512, 256, 24
    layer, host = build_layer(N, k, H, I, 5, fmt="bf16", int4_experts=range(N), with_router=False)
    x, xd = _x(5, B, H, "f32")
    logits = synth.logits(5, B, N, 1.0)
    _run_and_check(layer, host, x, xd, logits, "topk", 0, 1.0, TOL["int4"])
    _run_and_check(layer, host, x, xd, logits, "oea", 1, 1.0, TOL["int4"])


@pytest.mark.parametrize("fmt,x_dtype,H,I", [
    ("bf16", "bf16", 512, 256), ("bf16", "f32", 512, 256), ("f32", "f32", 256, 128),
    ("int4", "bf16", 512, 256), ("int4", "f32", 256, 384), ("mixed", "bf16", 640, 384),
    # fewer tile columns than the four column slices: bf16 3 (phase A) and 2 (phase B), INT4 1
    ("bf16", "bf16", 96, 64), ("int4", "bf16", 128, 128),
])
@pytest.mark.parametrize("B,k", [(1, 8), (2, 4), (8, 1), (1, 1), (1, 2), (6, 2), (20, 1)])
def test_small_batch_column_split(fmt, x_dtype, H, I, B, k):
    # calls with B*k <= 8 routed pairs split each item's input columns over
    # the waves of a workgroup and add the partial sums in LDS; larger calls
    # (6x2, 20x1 here) do so in a phase whose items fit the grid when no
    # expert has more than 16 tokens
    N = 16
    int4 = {"int4": range(N), "mixed": range(0, N, 2)}.get(fmt, [])
    layer, host = build_layer(N, k, H, I, 40 + B, fmt="f32" if fmt == "f32" else "bf16", int4_experts=int4,
                              with_router=False)
    x, xd = _x(41 + B, B, H, x_dtype)
    logits = synth.logits(42 + B, B, N, 1.0)
    tol = TOL["int4"] if int4 else TOL[fmt]
    _run_and_check(layer, host, x, xd, logits, "topk", 0, 1.0, tol)
    if k > 1:
        _run_and_check(layer, host, x, xd, logits, "oea", 1, 1.0, tol)


@pytest.mark.parametrize("fmt", ["bf16", "f32"])
@pytest.mark.parametrize("B,k", [(1, 4), (16, 4)])
def test_smallest_shapes(fmt, B, k):
    # H = I = 32: one tile column per row block in both phases (bf16), two
    # (fp32); B*k = 4 takes the column-split path, 64 the per-wave items
    N, H, I = 8, 32, 32
    layer, host = build_layer(N, k, H, I, 60 + B, fmt=fmt, with_router=False)
    x, xd = _x(61 + B, B, H, "bf16" if fmt == "bf16" else "f32")
    logits = synth.logits(62 + B, B, N, 1.0)
    _run_and_check(layer, host, x, xd, logits, "topk", 0, 1.0, TOL[fmt])
    _run_and_check(layer, host, x, xd, logits, "oea", 2, 1.0, TOL[fmt])


def test_publish_switches_version():
    # page "DynaExq" section 2.2: switching a handle changes the version the next call reads
    N, k, H, I, B = 8, 2, 256, 128, 6
    layer, host = build_layer(N, k, H, I, 5, fmt="bf16", with_router=False)
    x, xd = _x(5, B, H, "bf16")
    logits = synth.logits(5, B, N, 2.0)
    _run_and_check(layer, host, x, xd, logits, "topk", 0, 1.0, TOL["bf16"])
    e = 3
    mats = synth.expert_weights_bf16(5, e, H, I)
    qd, he = {}, dict(fmt=oracle.FMT_INT4)
    for name, m in zip(("gate", "up", "down"), mats):
        qd[name], qd["s_" + name] = moe.quantize_int4_g128(bf16_dev(m))
        he[name], he["s_" + name] = oracle.quantize_int4(m)
    layer.publish(e, moe.ExpertTensors.pack(moe.MOE_W_INT4_G128, qd["gate"], qd["up"], qd["down"],
                                            qd["s_gate"], qd["s_up"], qd["s_down"]))
    host = list(host)
    host[e] = he
    _run_and_check(layer, host, x, xd, logits, "topk", 0, 1.0, TOL["int4"])


def test_empty_routing_gives_zero_output():
    N, k, H, I, B = 8, 2, 256, 128, 3
    layer, _ = build_layer(N, k, H, I, 6, fmt="bf16", with_router=False)
    x, xd = _x(6, B, H, "bf16")
    buf = layer.buffers(B)
    buf.route["idx"].fill_(-1)
    buf.route["w"].zero_()
    moe.dispatch(buf.route["idx"], N, buf.disp)
    buf.y.fill_(7.0)
    layer.ffn(xd, buf)
    torch.cuda.synchronize()
    assert int(buf.disp["T"].item()) == 0
    assert torch.count_nonzero(buf.y).item() == 0


def test_ffn_repeat_runs_are_bit_identical():
    N, k, H, I, B = 32, 8, 512, 256, 16
    layer, _ = build_layer(N, k, H, I, 7, fmt="bf16", with_router=False)
    _, xd = _x(7, B, H, "bf16")
    logits = torch.from_numpy(synth.logits(7, B, N, 2.0)).to(DEV)
    y1 = layer.forward(xd, "topk", logits=logits).y.clone()
    y2 = layer.forward(xd, "topk", logits=logits).y.clone()
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("B", [1, 16])
def test_phase_timed_call_matches_the_ffn_call(B):
    # moe_expert_ffn_phase_events runs the same kernels: y bit for bit, and
    # the four events it records are in stream order with non-negative gaps
    # (B = 1 takes the column-split kernels, B = 16 the per-wave ones)
    N, k, H, I = 32, 8, 512, 256
    layer, _ = build_layer(N, k, H, I, 8, fmt="bf16", with_router=False)
    _, xd = _x(8, B, H, "bf16")
    logits = torch.from_numpy(synth.logits(8, B, N, 2.0)).to(DEV)
    buf = layer.forward(xd, "oea", 3, logits=logits)
    y_ref = buf.y.clone()
    y = torch.full_like(y_ref, float("nan"))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    moe.expert_ffn_phase_events(layer.table, N, H, I, xd, buf.route["idx"], buf.route["w"], buf.disp, y, buf.ws, ev)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
    gaps = [ev[i].elapsed_time(ev[i + 1]) for i in range(3)]
    assert all(g >= 0.0 for g in gaps), gaps


# ---------------------------------------------------------------------------
# Full-size layers, whole path from x (router GEMV on the GPU), in the launch
# configuration the benchmark times.
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def qwen30b():
    s = synth.SHAPES["qwen30b"]
    layer, host = build_layer(s["N"], s["k"], s["H"], s["I"], 30, fmt="bf16")
    return layer, host


def _routing_margin_ok(logits64, k):
    """Smallest gap between consecutive ranked logits near the cut; the GPU's
    fp32 logits must not be able to swap two experts there."""
    srt = -np.sort(-logits64, axis=1)
    return float(np.min(srt[:, :k + 1][:, :-1] - srt[:, 1:k + 1]))


@pytest.mark.parametrize("mode,k0", [("topk", 0), ("oea", 3), ("oea", 5)])
def test_qwen30b_layer_b16_full_path(qwen30b, mode, k0):
    layer, host = qwen30b
    B = 16
    x, xd = _x(31, B, layer.H, "bf16")
    buf = layer.forward(xd, mode, k0, 1.0)
    torch.cuda.synchronize()
    glog = buf.logits.cpu().numpy()
    ref_logits = oracle.router_logits(x.astype(np.float64), layer.w_r.cpu().numpy().astype(np.float64))
    assert np.abs(glog - ref_logits).max() < 1e-4
    assert _routing_margin_ok(ref_logits, layer.k) > 1e-4        # no near-tie the fp32 GEMV could flip
    ref = oracle.route(ref_logits.astype(np.float32), layer.k, oea=(mode == "oea"), k0=k0, p=1.0)
    assert np.array_equal(buf.route["idx"].cpu().numpy(), ref["idx"])
    assert int(buf.disp["T"].item()) == oracle.dispatch(ref["idx"], layer.N)["T"]
    yref = oracle.expert_ffn(host, layer.H, layer.I, x, ref["idx"], ref["w"])
    err, rms = max_err_over_rms(buf.y, yref)
    assert err <= TOL["bf16"] * rms, (err, rms)


@pytest.mark.parametrize("mode,k0,p", [("topk", 0, 1.0), ("oea", 5, 0.7)])
def test_qwen30b_layer_b128_zipf_full_width(qwen30b, mode, k0, p):
    # Zipf-hot experts carry more than 32 tokens (several token passes); the
    # oracle checks every token of the batch
    layer, host = qwen30b
    B = 128
    x, xd = _x(32, B, layer.H, "bf16")
    logits = (synth.logits(32, B, layer.N, 0.9) + synth.zipf_bias(layer.N, 1.1)[None, :]).astype(np.float32)
    buf, _ = _run_and_check(layer, host, x, xd, logits, mode, k0, p, TOL["bf16"])
    assert buf.disp["cnt"].cpu().numpy().max() > 32


@pytest.fixture(scope="module")
def qwen235b():
    s = synth.SHAPES["qwen235b"]
    layer, host = build_layer(s["N"], s["k"], s["H"], s["I"], 235, fmt="bf16")
    yield layer, host
    del layer, host
    torch.cuda.empty_cache()


@pytest.mark.parametrize("B", [16, 32, 64])
@pytest.mark.parametrize("mode,k0", [("topk", 0), ("oea", 5)])
def test_qwen235b_benchmark_points(qwen235b, B, mode, k0):
    # every Qwen3-235B-shaped point the benchmark reports, with its weights
    # (seed 235), router and first batch, through the whole layer (router
    # GEMV on the GPU); routing bit-exact where the GPU's fp32 logits cannot
    # flip a decision, the expert FFN on every token of the batch
    layer, host = qwen235b
    print(f"qwen235b B={B} {mode} k0={k0}", flush=True)
    x, xd = _x(400, B, layer.H, "bf16")
    buf = layer.forward(xd, mode, k0, 1.0)
    torch.cuda.synchronize()
    glog = buf.logits.cpu().numpy()
    ref32 = oracle.router_logits(x.astype(np.float64), layer.w_r.cpu().numpy().astype(np.float64)).astype(np.float32)
    eps = float(np.abs(glog.astype(np.float64) - ref32).max())
    assert eps < 1e-4
    ref = oracle.route(ref32, layer.k, oea=(mode == "oea"), k0=k0, p=1.0)
    assert routing_order_is_robust(ref32, ref["idx"], eps)
    assert np.array_equal(buf.route["idx"].cpu().numpy(), ref["idx"])
    assert np.abs(buf.route["w"].cpu().numpy().astype(np.float64) - ref["w"]).max() <= 1e-6
    dref = oracle.dispatch(ref["idx"], layer.N)
    for key in ("cnt", "offsets", "perm", "active"):
        assert np.array_equal(buf.disp[key].cpu().numpy(), dref[key]), key
    assert int(buf.disp["T"].item()) == dref["T"]
    yref = oracle.expert_ffn(host, layer.H, layer.I, x, ref["idx"], ref["w"])
    err, rms = max_err_over_rms(buf.y, yref)
    assert err <= TOL["bf16"] * rms, (err, rms)


@pytest.fixture(scope="module")
def mixed_hot_set():
    # the benchmark's hot set: the EMA (alpha 0.9) of vanilla top-8 dispatch
    # counts over 64 Zipf-biased B=32 batches (seeds 200..263) of the
    # Qwen3-30B-shaped layer's router (seed 30)
    s = synth.SHAPES["qwen30b"]
    N, k, H = s["N"], s["k"], s["H"]
    B, warm = 32, 64
    bias = synth.zipf_bias(N, 1.1)
    w_r = synth.router_weight(30, N, H)
    xbits = [synth.to_bf16_bits(synth.activations(200 + b, B, H)) for b in range(warm)]
    hot = moe.ema_hot_set([bf16_dev(xb) for xb in xbits], torch.from_numpy(w_r).to(DEV),
                          torch.from_numpy(bias).to(DEV), k, 32, 0.9)
    return hot, xbits, bias, w_r


def test_mixed_hot_set_equals_the_oracles(mixed_hot_set):
    # the same EMA from the oracle's own router logits, routing and dispatch
    hot, xbits, bias, w_r = mixed_hot_set
    N = w_r.shape[0]
    S = np.zeros(N)
    for xb in xbits:
        lg = (oracle.router_logits(synth.bf16_bits_to_f32(xb).astype(np.float64), w_r.astype(np.float64))
              + bias[None, :].astype(np.float64)).astype(np.float32)
        r = oracle.route(lg, 8, oea=False)
        S = oracle.hotness_ema(S, oracle.dispatch(r["idx"], N)["cnt"], 0.9)
    assert hot == sorted(np.argsort(-S, kind="stable")[:32].tolist())


@pytest.mark.parametrize("mode,k0", [("topk", 0), ("oea", 5)])
def test_qwen30b_mixed_int4_b32_as_benchmarked(mixed_hot_set, mode, k0):
    # the mixed-residency layer exactly as the benchmark builds it: the EMA
    # hot set in bf16, the other 96 experts INT4 group-128, B = 32 on the
    # benchmark's first batch (seed 300) with Zipf-biased router logits; the
    # oracle computes every token with the dequantised INT4 weights
    hot, _, bias, w_r = mixed_hot_set
    s = synth.SHAPES["qwen30b"]
    cold = [e for e in range(s["N"]) if e not in set(hot)]
    layer, host = build_layer(s["N"], s["k"], s["H"], s["I"], 30, fmt="bf16", int4_experts=cold,
                              with_router=False)
    B = 32
    x, xd = _x(300, B, layer.H, "bf16")
    logits = (oracle.router_logits(x.astype(np.float64), w_r.astype(np.float64))
              + bias[None, :].astype(np.float64)).astype(np.float32)
    ref = oracle.route(logits, layer.k, oea=(mode == "oea"), k0=k0, p=1.0)
    _, rel = _run_and_check(layer, host, x, xd, logits, mode, k0, 1.0, TOL["int4"])
    assert any(e in cold for e in ref["idx"].ravel()) and any(e in hot for e in ref["idx"].ravel())
    del layer
    torch.cuda.empty_cache()
