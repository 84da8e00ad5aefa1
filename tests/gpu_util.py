"""Helpers shared by the GPU parity tests: build a layer on the device from the
seeded generators and keep host copies of the same weights for the oracle."""
from __future__ import annotations

import numpy as np
import torch

import aware_expert_routing_amd as moe
import oracle
import synth

DEV = torch.device("cuda:0")


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def u16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV)


def build_layer(N, k, H, I, seed, fmt="bf16", int4_experts=(), with_router=True):
    """Returns (layer, host_experts) where host_experts is the oracle's view.

    fmt 'f32' or 'bf16' for every expert; experts listed in int4_experts are
    quantised on the GPU (moe_quantize_int4_g128) and, independently, by the
    oracle's quantiser for the host copy.
    """
    host, dev = [], []
    rowmajor_int4 = {}   # the quantiser's row-major output per INT4 expert, before packing
    int4 = set(int4_experts)
    for e in range(N):
        if fmt == "f32":
            g, u, d = synth.expert_weights_f32(seed, e, H, I)
            host.append(dict(fmt=oracle.FMT_F32, gate=g, up=u, down=d))
            dev.append(moe.ExpertTensors.pack(moe.MOE_W_F32, torch.from_numpy(g).to(DEV),
                                              torch.from_numpy(u).to(DEV), torch.from_numpy(d).to(DEV)))
            continue
        mats = synth.expert_weights_bf16(seed, e, H, I)
        if e in int4:
            he = dict(fmt=oracle.FMT_INT4)
            qd = {}
            for name, m in zip(("gate", "up", "down"), mats):
                q, s = oracle.quantize_int4(m)
                he[name], he["s_" + name] = q, s
                gq, gs = moe.quantize_int4_g128(bf16_dev(m))
                qd[name], qd["s_" + name] = gq, gs
            host.append(he)
            rowmajor_int4[e] = qd
            dev.append(moe.ExpertTensors.pack(moe.MOE_W_INT4_G128, qd["gate"], qd["up"], qd["down"],
                                              qd["s_gate"], qd["s_up"], qd["s_down"]))
        else:
            host.append(dict(fmt=oracle.FMT_BF16, gate=mats[0], up=mats[1], down=mats[2]))
            dev.append(moe.ExpertTensors.pack(moe.MOE_W_BF16, *[bf16_dev(m) for m in mats]))
    w_r = None
    if with_router:
        w_r = torch.from_numpy(synth.router_weight(seed, N, H)).to(DEV)
    layer = moe.MoELayer(H, I, N, k, w_r, dev, DEV)
    layer.rowmajor_int4 = rowmajor_int4
    torch.cuda.synchronize()
    return layer, host


def max_err_over_rms(y_gpu: torch.Tensor, y_ref: np.ndarray):
    y = y_gpu.detach().cpu().numpy().astype(np.float64)
    rms = float(np.sqrt(np.mean(y_ref ** 2)))
    err = float(np.abs(y - y_ref).max())
    return err, rms


def gamma(n: int, u: float = 2.0 ** -24) -> float:
    """Standard bound on the relative error of an n-term floating-point sum."""
    return n * u / (1.0 - n * u)


def routing_order_is_robust(logits32: np.ndarray, ref_idx: np.ndarray, eps: float) -> bool:
    """True when no routing decision can differ between two logit matrices
    that differ by at most eps elementwise: for every token, the logits at
    consecutive rank positions 0 .. d+1 (d = the deepest rank the routing
    took, so every comparison the selection made lies inside) are more than
    2 eps apart.  Lets a test route with the oracle on its own logits and
    still demand bit-exact indices from the GPU's router output."""
    B, N = logits32.shape
    for i in range(B):
        order = np.lexsort((np.arange(N), -logits32[i].astype(np.float64)))
        pos = np.empty(N, np.int64)
        pos[order] = np.arange(N)
        sel = [int(e) for e in ref_idx[i] if e >= 0]
        depth = int(max(pos[e] for e in sel)) if sel else 0
        l = logits32[i][order[:min(N, depth + 2)]].astype(np.float64)
        if l.size > 1 and np.min(l[:-1] - l[1:]) <= 2.0 * eps:
            return False
    return True

