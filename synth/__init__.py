"""Seeded synthetic inputs for the decode MoE layer.

This module serves both the GPU library's tests/benchmark and the CPU oracle's
tests.  It holds none of the method's arithmetic: it draws seeded normal
values (numpy PCG64), encodes them as bf16 (round to nearest even), and builds
the per-expert logit bias that mimics heavy-tailed routing.

Workload recipes (shapes follow the Qwen3-30B-A3B / Qwen3-235B-A22B MoE layers
named on the OEA page, section 2 Q3; N = 128 experts, top-8):
  * ``tiny``      N=16, k=4, H=256, I=128, B=4, fp32, logits ~N(0,1) given directly.
  * ``qwen30b``   H=2048, I=768, N=128, k=8, bf16 experts ~N(0,0.02),
                  router W_r [128,2048] fp32 ~N(0,0.02), x ~N(0,1) bf16.
  * ``qwen235b``  H=4096, I=1536, otherwise as ``qwen30b``.
Zipf routing bias: beta_e = -s * ln(r_e) with r a seeded permutation of 1..N
(the log of a Zipf(s) prior, added to the router logits); s = 0 is the uniform
control.
"""
from __future__ import annotations

import numpy as np

SHAPES = {
    "tiny": dict(N=16, k=4, H=256, I=128),
    "qwen30b": dict(N=128, k=8, H=2048, I=768),
    "qwen235b": dict(N=128, k=8, H=4096, I=1536),
}

WEIGHT_STD = 0.02


def rng(*key: int) -> np.random.Generator:
    """A PCG64 generator keyed by a tuple of non-negative integers."""
    return np.random.default_rng(np.random.SeedSequence([int(v) for v in key]))


def normal(key, shape, std: float = 1.0) -> np.ndarray:
    """float32 N(0, std^2) samples for a key tuple."""
    if isinstance(key, int):
        key = (key,)
    a = rng(*key).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    nan = np.isnan(a)
    r = r.astype(np.uint16)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def zipf_bias(N: int, s: float, seed: int = 7) -> np.ndarray:
    """beta_e = -s * ln(r_e), r a seeded permutation of 1..N (float32)."""
    if s == 0:
        return np.zeros(N, np.float32)
    r = rng(seed, N).permutation(N) + 1
    return (-s * np.log(r.astype(np.float64))).astype(np.float32)


def expert_weights_bf16(layer_seed: int, e: int, H: int, I: int):
    """bf16 bit patterns for one expert: gate [I,H], up [I,H], down [H,I], ~N(0, 0.02)."""
    g = to_bf16_bits(normal((layer_seed, e, 0), (I, H), WEIGHT_STD))
    u = to_bf16_bits(normal((layer_seed, e, 1), (I, H), WEIGHT_STD))
    d = to_bf16_bits(normal((layer_seed, e, 2), (H, I), WEIGHT_STD))
    return g, u, d


def expert_weights_f32(layer_seed: int, e: int, H: int, I: int):
    g = normal((layer_seed, e, 0), (I, H), WEIGHT_STD)
    u = normal((layer_seed, e, 1), (I, H), WEIGHT_STD)
    d = normal((layer_seed, e, 2), (H, I), WEIGHT_STD)
    return g, u, d


def router_weight(layer_seed: int, N: int, H: int) -> np.ndarray:
    return normal((layer_seed, 1_000_000), (N, H), WEIGHT_STD)


def activations(batch_seed: int, B: int, H: int) -> np.ndarray:
    """x ~ N(0,1) as float32 (callers encode to bf16 where the workload says so)."""
    return normal((batch_seed, 2_000_000), (B, H))


def logits(batch_seed: int, B: int, N: int, scale: float = 1.0) -> np.ndarray:
    """Directly-given router logits ~ N(0,1) * scale (float32)."""
    return normal((batch_seed, 3_000_000), (B, N)) * np.float32(scale)


def tied_logits(batch_seed: int, B: int, N: int, levels: int = 4) -> np.ndarray:
    """Logits drawn from a few distinct values so that many exact ties occur."""
    v = rng(batch_seed, 4_000_000).integers(0, levels, size=(B, N)).astype(np.float32)
    return v * np.float32(0.5)
