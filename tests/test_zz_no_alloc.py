"""moe_expert_ffn_noalloc (the expert FFN on the library's static workspace,
for callers that cannot allocate) against moe_expert_ffn on the same inputs:
two calls in a row, the second smaller, each bit-identical to the
workspace-taking entry point (the same kernels and launch shapes), and the
small call also within the bf16 bar of the CPU oracle."""
import numpy as np
import pytest
import torch

import aware_expert_routing_amd as moe
import oracle
import synth
from gpu_util import DEV, bf16_dev, build_layer, max_err_over_rms

pytestmark = pytest.mark.gpu


def _route(layer, B, seed, scale=1.0, zipf=0.0):
    logits = (synth.logits(seed, B, layer.N, scale) + synth.zipf_bias(layer.N, zipf)[None, :]).astype(np.float32)
    xb = synth.to_bf16_bits(synth.activations(seed, B, layer.H))
    buf = layer.buffers(B)
    layer.route(torch.from_numpy(logits).to(DEV), "topk", 0, 1.0, buf)
    return logits, synth.bf16_bits_to_f32(xb), bf16_dev(xb), buf


def test_noalloc_matches_the_workspace_entry_point():
    s = synth.SHAPES["qwen30b"]
    layer, host = build_layer(s["N"], s["k"], s["H"], s["I"], 30, fmt="bf16", with_router=False)
    # B = 64 with Zipf routing (hot experts with more than 16 tokens), then
    # B = 3 (the small-batch column-split kernels) on the same static array
    for B, seed, zipf in ((64, 90, 1.1), (3, 91, 0.0)):
        print(f"noalloc case B={B} seed={seed}", flush=True)
        logits, x, xd, buf = _route(layer, B, seed, zipf=zipf)
        y_ref = layer.ffn(xd, buf).clone()
        y = torch.full((B, layer.H), float("nan"), device=DEV)
        moe.expert_ffn_noalloc(layer.table, layer.N, layer.H, layer.I, xd, buf.route["idx"], buf.route["w"],
                               buf.disp, y)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), B
        if B <= 8:
            ref = oracle.route(logits, layer.k, oea=False)
            assert np.array_equal(buf.route["idx"].cpu().numpy(), ref["idx"])
            yref = oracle.expert_ffn(host, layer.H, layer.I, x, ref["idx"], ref["w"])
            err, rms = max_err_over_rms(y, yref)
            assert err <= 1e-2 * rms, (err, rms)
    # the workspace-taking entry point is unaffected by the static array's use
    y_again = layer.ffn(xd, buf).clone()
    torch.cuda.synchronize()
    assert torch.equal(y_again, y)
    del layer
    torch.cuda.empty_cache()


def test_noalloc_refuses_calls_beyond_the_static_workspace():
    N, k, H, I, B = 16, 16, 4096, 1536, 128
    assert moe.ffn_workspace_bytes(B, k, H, I) > moe.NOALLOC_WORKSPACE_BYTES
    i32 = dict(device=DEV, dtype=torch.int32)
    table = torch.zeros(N * moe.HANDLE_BYTES, dtype=torch.uint8, device=DEV)
    x = torch.zeros(B, H, device=DEV, dtype=torch.bfloat16)
    idx = torch.zeros(B, k, **i32)
    w = torch.zeros(B, k, device=DEV)
    disp = dict(offsets=torch.zeros(N + 1, **i32), perm=torch.zeros(B * k, **i32), active=torch.zeros(N, **i32),
                T=torch.zeros(1, **i32))
    y = torch.zeros(B, H, device=DEV)
    with pytest.raises(moe.MoeError) as ei:
        moe.expert_ffn_noalloc(table, N, H, I, x, idx, w, disp, y)
    assert ei.value.status == -2
