"""A decode MoE layer assembled from the libmoe entry points.

The layer owns device weights, the per-expert handle table (page "DynaExq",
section 2.2: stable handles resolved at run time) and preallocated buffers,
so a forward call enqueues kernels only: router logits -> vanilla top-k or
OEA routing (page "Opportunistic Expert Activation (OEA) - L2", section 2 Q2)
-> dispatch -> expert FFN with weighted combine.  T and every size that
depends on the routing stay on the device.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

from . import _lib as L


@dataclass
class ExpertTensors:
    """One expert version in the packed layout the FFN reads (moe_pack_weights)."""
    fmt: int
    gate: torch.Tensor
    up: torch.Tensor
    down: torch.Tensor
    s_gate: torch.Tensor | None = None
    s_up: torch.Tensor | None = None
    s_down: torch.Tensor | None = None

    @classmethod
    def pack(cls, fmt: int, gate, up, down, s_gate=None, s_up=None, s_down=None, stream=None):
        """Pack row-major device matrices ([I,H], [I,H], [H,I]; INT4: the
        quantiser's bytes and scales) into a new version."""
        g, sg = L.pack_weights(fmt, gate, s_gate, stream=stream)
        u, su = L.pack_weights(fmt, up, s_up, stream=stream)
        d, sd = L.pack_weights(fmt, down, s_down, stream=stream)
        return cls(fmt, g, u, d, sg, su, sd)

    def handle(self) -> L.ExpertHandle:
        h = L.ExpertHandle()
        h.fmt = self.fmt
        h.group = 128 if self.fmt == L.MOE_W_INT4_G128 else 0
        h.w_gate, h.w_up, h.w_down = self.gate.data_ptr(), self.up.data_ptr(), self.down.data_ptr()
        if self.fmt == L.MOE_W_INT4_G128:
            h.s_gate, h.s_up, h.s_down = self.s_gate.data_ptr(), self.s_up.data_ptr(), self.s_down.data_ptr()
        h.reserved = 0
        return h


@dataclass
class Buffers:
    """Per-batch-size device buffers for one forward call.

    route: idx [B, k] and w [B, k] (the routing result), n_base [B] and mask
    [ceil(N/32)] (OEA and pruned modes only: the baseline counts and S_base;
    vanilla top-k leaves them as they were), T [1] (the same tensor as
    disp["T"]).  disp: cnt, offsets, perm, active, T (dispatch output).
    y: [B, H] layer output.  ws: the expert FFN's workspace.  extra["sync"]:
    the fused router kernel's completion counter (zero between calls)."""
    B: int
    logits: torch.Tensor
    route: dict
    disp: dict
    y: torch.Tensor
    ws: torch.Tensor
    extra: dict = field(default_factory=dict)


class MoELayer:
    def __init__(self, H: int, I: int, N: int, k: int, w_r: torch.Tensor | None,
                 experts: list[ExpertTensors], device="cuda"):
        self.H, self.I, self.N, self.k = H, I, N, k
        self.w_r = w_r
        self.experts = list(experts)
        self.device = torch.device(device)
        self.table = torch.zeros(N * L.HANDLE_BYTES, dtype=torch.uint8, device=self.device)
        for e, ex in enumerate(self.experts):
            L.handle_publish(self.table, e, ex.handle())
        self._bufs: dict[int, Buffers] = {}

    def publish(self, e: int, ex: ExpertTensors, stream=None):
        """Point expert e at a new weight version (ordered on the stream)."""
        self.experts[e] = ex
        L.handle_publish(self.table, e, ex.handle(), stream)

    def buffers(self, B: int) -> Buffers:
        b = self._bufs.get(B)
        if b is None:
            dev, N, k = self.device, self.N, self.k
            i32 = dict(device=dev, dtype=torch.int32)
            T = torch.empty(1, **i32)   # written by dispatch; the routing result shares it
            route = dict(idx=torch.empty(B, k, **i32), w=torch.empty(B, k, device=dev, dtype=torch.float32),
                         n_base=torch.empty(B, **i32), mask=torch.empty((N + 31) // 32, **i32), T=T)
            disp = dict(cnt=torch.empty(N, **i32), offsets=torch.empty(N + 1, **i32),
                        perm=torch.empty(B * k, **i32), active=torch.empty(N, **i32), T=T)
            ws = torch.zeros(L.ffn_workspace_bytes(B, k, self.H, self.I), device=dev, dtype=torch.uint8)
            b = Buffers(B, torch.empty(B, N, device=dev, dtype=torch.float32), route, disp,
                        torch.empty(B, self.H, device=dev, dtype=torch.float32), ws,
                        {"sync": torch.zeros(1, **i32)})
            self._bufs[B] = b
        return b

    def route(self, logits: torch.Tensor, mode: str, k0: int = 0, p: float = 1.0,
              buf: Buffers | None = None, stream=None, max_p: int | None = None, n_valid=None,
              k0_by_batch=None) -> Buffers:
        """Routing ("topk", "oea" or "pruned") and dispatch (one launch up to 48 tokens); n_valid
        (device int32 [1]) marks trailing tokens as padding; k0_by_batch (device
        int32 [B+1], see k0_schedule) picks k0 from the real batch size."""
        B = logits.shape[0]
        buf = buf or self.buffers(B)
        if mode not in ("topk", "oea", "pruned"):
            raise ValueError(mode)
        L.route_dispatch(logits, self.k, mode, k0, p, True, buf.route, buf.disp, stream, max_p, n_valid,
                         k0_by_batch, buf.extra["sync"])
        return buf

    def ffn(self, x: torch.Tensor, buf: Buffers, stream=None) -> torch.Tensor:
        return L.expert_ffn(self.table, self.N, self.H, self.I, x, buf.route["idx"], buf.route["w"],
                            buf.disp, buf.y, buf.ws, stream)

    def forward(self, x: torch.Tensor, mode: str = "oea", k0: int = 3, p: float = 1.0,
                logits: torch.Tensor | None = None, stream=None, max_p: int | None = None,
                n_valid=None, k0_by_batch=None) -> Buffers:
        """Whole layer.  If `logits` is given the router GEMV is skipped;
        otherwise router, routing and dispatch run together (one launch up to 48
        tokens)."""
        B = x.shape[0]
        buf = self.buffers(B)
        stream = L._stream(stream)   # looked up once for both calls
        if logits is None:
            if mode not in ("topk", "oea", "pruned"):
                raise ValueError(mode)
            L.router_route_dispatch(x, self.w_r, self.k, mode, k0, p, True, buf.route, buf.disp, buf.logits,
                                    buf.extra["sync"], stream, max_p, n_valid, k0_by_batch)
        else:
            self.route(logits, mode, k0, p, buf, stream, max_p, n_valid, k0_by_batch)
        self.ffn(x, buf, stream)
        return buf

    def capture(self, x: torch.Tensor, mode: str = "oea", k0: int = 3, p: float = 1.0,
                max_p: int | None = None, n_valid=None, k0_by_batch=None) -> torch.cuda.CUDAGraph:
        """Capture forward(x, ...) into a HIP graph (every kernel of the layer, no
        allocation or memset inside).  Replaying it recomputes the layer for
        whatever `x` and `n_valid` hold at replay time; results land in
        self.buffers(B).  Pair it with `n_valid` to serve real batches smaller
        than B without padding tokens inflating T."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):   # warm-up outside capture (allocates the buffers)
            self.forward(x, mode, k0, p, max_p=max_p, n_valid=n_valid, k0_by_batch=k0_by_batch)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.forward(x, mode, k0, p, max_p=max_p, n_valid=n_valid, k0_by_batch=k0_by_batch)
        return graph


def capture_layers(calls, mode: str = "oea", k0: int = 3, p: float = 1.0, max_p: int | None = None,
                   n_valid=None, k0_by_batch=None) -> torch.cuda.CUDAGraph:
    """Capture the forward calls of several layers, in the order given, into
    one HIP graph; `calls` is a list of (MoELayer, x) pairs.  One replay runs
    them all (a decode step's MoE layers), so the fixed cost of launching a
    graph is paid once per step rather than once per layer, and the host
    spends one replay call on the whole step.  Each layer's results land in
    its own buffers(B), as with MoELayer.capture."""
    calls = list(calls)
    if not calls:
        raise ValueError("no layers to capture")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up outside capture (allocates every layer's buffers)
        for layer, x in calls:
            layer.forward(x, mode, k0, p, max_p=max_p, n_valid=n_valid, k0_by_batch=k0_by_batch)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for layer, x in calls:
            layer.forward(x, mode, k0, p, max_p=max_p, n_valid=n_valid, k0_by_batch=k0_by_batch)
    return graph


def k0_schedule(k: int, B_max: int, steps: list[tuple[int, int]], device="cuda") -> torch.Tensor:
    """Device table for moe_route_dispatch's k0_by_batch: entry b is the k0
    for a batch of b real tokens.

    Page "Opportunistic Expert Activation (OEA) - L2", section 7 implementation notes:
    piggybacking cannot help a single token, and the natural tuning axis is a
    batch-size-dependent k0, larger (safer) at small B.  `steps` lists
    (first batch size, k0) pairs in increasing batch size; batch sizes below
    the first pair, and B = 1 always, use k0 = k (plain top-k routing).
    """
    table = [k] * (B_max + 1)
    for b0, k0 in sorted(steps):
        if not 1 <= k0 <= k:
            raise ValueError("k0 must be in [1, k]")
        for b in range(max(b0, 2), B_max + 1):
            table[b] = k0
    return torch.tensor(table, dtype=torch.int32, device=device)
