"""Seeded random sweep of the whole path against the oracle: random layer
sizes, expert formats (all fp32, or bf16 with a random INT4 subset),
activation dtype, routing mode and knobs, batch size and logit scale, with
and without the router GEMV, with a random max-rank limit and random
trailing padding tokens.

Each case checks the routing bit for bit (idx, T) and the weights within
1e-6 on the logits the layer used, and the layer output within the loosest
tolerance of the formats present (1e-4 fp32, 1e-2 bf16, 2e-2 with INT4).
Page "Opportunistic Expert Activation (OEA) - L2", sections 2-4; page
"DynaExq", sections 2.2 / 3.2 (per-expert versions in one layer).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, bf16_dev, build_layer, max_err_over_rms

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 1e-2, "int4": 2e-2}


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    N = int(rng.choice([1, 3, 8, 16, 37, 64, 128]))
    k = int(rng.integers(1, min(N, 16) + 1))
    fmt = "f32" if rng.random() < 0.2 else "bf16"
    # multiples of 128 keep every format legal (INT4 groups of 128)
    H = 128 * int(rng.integers(1, 5))
    I = 128 * int(rng.integers(1, 5))
    B = int(rng.choice([1, 2, 5, 16, 17, 33, 64, 128]))
    int4 = [] if fmt == "f32" else [e for e in range(N) if rng.random() < 0.4]
    mode = str(rng.choice(["topk", "oea", "pruned"]))
    k0 = int(rng.integers(1, k + 1))
    p = float(rng.choice([1.0, 0.9, 0.6]))
    scale = float(rng.choice([0.5, 1.0, 4.0]))
    zipf = bool(rng.random() < 0.5)
    x_dtype = "f32" if (fmt == "f32" or rng.random() < 0.25) else "bf16"
    router = bool(rng.random() < 0.5)
    max_p = int(rng.integers(k, N + 1)) if (mode == "oea" and rng.random() < 0.3) else None
    n_valid = int(rng.integers(0, B + 1)) if rng.random() < 0.25 else None   # trailing padding tokens
    return dict(N=N, k=k, fmt=fmt, H=H, I=I, B=B, int4=int4, mode=mode, k0=k0, p=p, scale=scale,
                zipf=zipf, x_dtype=x_dtype, router=router, max_p=max_p, n_valid=n_valid)


@pytest.mark.parametrize("seed", range(48))
def test_random_layer_against_oracle(seed):
    c = _case(seed)
    print("case", seed, c, flush=True)
    N, k, H, I, B = c["N"], c["k"], c["H"], c["I"], c["B"]
    layer, host = build_layer(N, k, H, I, 50 + seed, fmt=c["fmt"], int4_experts=c["int4"], with_router=c["router"])
    x = synth.activations(60 + seed, B, H)
    if c["x_dtype"] == "bf16":
        xb = synth.to_bf16_bits(x)
        x, xd = synth.bf16_bits_to_f32(xb), bf16_dev(xb)
    else:
        xd = torch.from_numpy(x).to(DEV)
    mode, k0, p, max_p, nv = c["mode"], c["k0"], c["p"], c["max_p"], c["n_valid"]
    n_valid = None if nv is None else torch.tensor([nv], dtype=torch.int32, device=DEV)
    if c["router"]:
        buf = layer.forward(xd, mode, k0, p, max_p=max_p, n_valid=n_valid)
    else:
        logits = synth.logits(70 + seed, B, N, c["scale"])
        if c["zipf"]:
            logits = (logits + synth.zipf_bias(N, 1.1)[None, :]).astype(np.float32)
        buf = layer.forward(xd, mode, k0, p, logits=torch.from_numpy(logits).to(DEV), max_p=max_p, n_valid=n_valid)
    torch.cuda.synchronize()
    l = buf.logits.cpu().numpy() if c["router"] else logits
    ref = oracle.route(l, k, oea=(mode != "topk"), k0=k0, p=p, pruned=(mode == "pruned"), max_p=max_p,
                       n_valid=nv)
    assert np.array_equal(buf.route["idx"].cpu().numpy(), ref["idx"])
    assert np.abs(buf.route["w"].cpu().numpy().astype(np.float64) - ref["w"]).max() <= 1e-6
    assert int(buf.disp["T"].item()) == len(set(ref["idx"][ref["idx"] >= 0].tolist()))
    assert int(buf.route["T"].item()) == int(buf.disp["T"].item())   # the routing result reports the same T
    yref = oracle.expert_ffn(host, H, I, x, ref["idx"], ref["w"])
    if not np.any(ref["idx"] >= 0):   # every token is padding: the output is exactly zero
        assert not torch.any(buf.y).item()
        return
    err, rms = max_err_over_rms(buf.y, yref)
    tol = TOL["int4"] if c["int4"] else TOL[c["fmt"]]
    assert err <= tol * rms + 1e-30, (err, rms, err / max(rms, 1e-30))
