"""Online precision residency for one MoE layer (page "DynaExq", sections
2.2-2.5 / 3.2-3.5), on top of the libmoe residency entry points
(include/moe_residency.h).

The object owns the device memory the C library only manages: the pool arena
for high-precision versions, the score and counter vectors, the pinned score
copy, and a migration stream (default priority) for the host-to-device
copies.  The C library keeps the state machine, the pool's free list, the
budget tracker and the policy; this module marshals arguments.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib as L
from .layer import ExpertTensors, MoELayer


def pinned_hi_version(ex: ExpertTensors) -> torch.Tensor:
    """Copy a packed bf16 version (device) into one pinned host buffer laid
    out gate | up | down, the form the residency manager copies in."""
    if ex.fmt != L.MOE_W_BF16:
        raise ValueError("the high-precision version must be bf16")
    parts = [t.reshape(-1).view(torch.uint8) for t in (ex.gate, ex.up, ex.down)]
    out = torch.empty(sum(p.numel() for p in parts), dtype=torch.uint8, pin_memory=True)
    o = 0
    for p in parts:
        out[o:o + p.numel()].copy_(p)
        o += p.numel()
    return out


class Residency:
    """High-precision residency manager for `layer`.

    lo      : the resident low-precision version of every expert; the layer's
              table must hold these when the manager is created
    hi_host : [N] pinned host buffers from pinned_hi_version
    n_hi    : high-precision capacity (experts); the pool gets pool_blocks
              blocks (default n_hi) and the budget budget_bytes (default the
              whole pool)
    """

    def __init__(self, layer: MoELayer, lo: list[ExpertTensors], hi_host: list[torch.Tensor], n_hi: int,
                 alpha: float = 0.9, margin: float = 0.0, interval_s: float = -1.0,
                 pool_blocks: int | None = None, budget_bytes: int | None = None, stream=None):
        N, H, I = layer.N, layer.H, layer.I
        if len(lo) != N or len(hi_host) != N:
            raise ValueError("lo and hi_host need one entry per expert")
        self.layer = layer
        self.N = N
        self.hi_bytes = 6 * H * I
        self.block_bytes = (self.hi_bytes + 255) // 256 * 256
        nblk = n_hi if pool_blocks is None else pool_blocks
        dev = layer.device
        self.arena = torch.empty(max(nblk, 1) * self.block_bytes, dtype=torch.uint8, device=dev)
        self.S = torch.zeros(N, dtype=torch.float32, device=dev)
        self.c = torch.zeros(N, dtype=torch.int32, device=dev)
        self.S_host = torch.zeros(N, dtype=torch.float32, pin_memory=True)
        self.compute = torch.cuda.current_stream(dev) if stream is None else stream
        self.mig = torch.cuda.Stream(device=dev)          # default priority
        self.lo = list(lo)
        self.hi_host = list(hi_host)
        self._lo_arr = (L.ExpertHandle * N)(*[x.handle() for x in self.lo])
        self._src_arr = (ctypes.c_void_p * N)(*[t.data_ptr() for t in self.hi_host])
        self.pool = L.pool_create(self.arena.data_ptr(), self.arena.numel(), self.block_bytes)
        total = self.arena.numel() if budget_bytes is None else budget_bytes
        self.budget = L.budget_create(total, 0)
        cfg = L.ResidencyConfig()
        cfg.N, cfg.H, cfg.I = N, H, I
        cfg.table = layer.table.data_ptr()
        cfg.lo = self._lo_arr
        cfg.hi_src = self._src_arr
        cfg.pool_hi, cfg.budget = self.pool, self.budget
        cfg.S, cfg.c, cfg.S_host = self.S.data_ptr(), self.c.data_ptr(), self.S_host.data_ptr()
        cfg.n_hi, cfg.alpha, cfg.margin, cfg.interval_s = n_hi, alpha, margin, interval_s
        cfg.compute_stream, cfg.mig_stream = self.compute.cuda_stream, self.mig.cuda_stream
        self.cfg = cfg
        try:
            self.handle = L.residency_create(cfg)
        except Exception:
            L.lib().moe_pool_destroy(self.pool)
            L.lib().moe_budget_destroy(self.budget)
            raise

    def step(self, cnt: torch.Tensor | None = None, force: bool = False, wait: bool = False):
        """A window boundary after a forward call whose dispatch counts are cnt."""
        L.residency_step(self.handle, cnt, force=force, wait=wait)

    def state(self, e: int) -> int:
        return L.lib().moe_residency_state(self.handle, e)

    def states(self) -> list[int]:
        return [self.state(e) for e in range(self.N)]

    def hi_set(self) -> set[int]:
        """Experts whose published version is the high-precision one."""
        return {e for e, s in enumerate(self.states()) if s == L.MOE_RES_HI}

    def pending(self) -> int:
        return L.lib().moe_residency_pending(self.handle)

    def stats(self) -> dict:
        return L.residency_stats(self.handle)

    def budget_used(self) -> int:
        return L.lib().moe_budget_used(self.budget)

    def free_blocks(self) -> int:
        return L.lib().moe_pool_free_blocks(self.pool)

    def close(self):
        """Switch every expert back to its low-precision version, wait for the
        layer's stream, and free the manager (the arena may then go)."""
        if getattr(self, "handle", None):
            for e, st in enumerate(self.states()):
                if st != L.MOE_RES_LO:
                    L.handle_publish(self.layer.table, e, self.lo[e].handle(), self.compute)
            self.compute.synchronize()
            L._check("moe_residency_destroy", L.lib().moe_residency_destroy(self.handle))
            self.handle = None
            L.lib().moe_pool_destroy(self.pool)
            L.lib().moe_budget_destroy(self.budget)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def ema_hot_set(xs, w_r: torch.Tensor, bias: torch.Tensor, k: int, n_hot: int, alpha: float = 0.9,
                stream=None) -> list[int]:
    """A static high-precision set from routing history (page "DynaExq",
    section 2.5: per-expert counts folded into S <- alpha S + (1 - alpha) c;
    section 2.5 / 3.5: the top-n_hi experts by S).

    For each batch x in `xs` (in order): router logits (moe_router_logits)
    plus the per-expert `bias`, vanilla top-k routing and dispatch
    (moe_route_dispatch), and the hotness update (moe_hotness_ema) on the
    dispatch counts, starting from S = 0.  Returns the n_hot experts with the
    largest S, ties to the lower index, in ascending expert order.
    """
    N = w_r.shape[0]
    S = torch.zeros(N, device=w_r.device, dtype=torch.float32)
    for x in xs:
        logits = L.router_logits(x, w_r, stream=stream) + bias[None, :]
        _, disp = L.route_dispatch(logits, k, "topk", stream=stream)
        L.hotness_ema(S, disp["cnt"], alpha, stream=stream)
    order = torch.argsort(S.cpu(), descending=True, stable=True)
    return sorted(int(e) for e in order[:n_hot])
