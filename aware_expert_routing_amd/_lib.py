"""ctypes binding of libmoe (the C ABI declared in include/moe.h).

Argument marshalling only: every function passes device pointers, sizes and
the current HIP stream straight to the library and raises on a non-zero
status.  Nothing here computes any part of the layer; if the built library
is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_LIB selects another build of the same library (e.g. the host-sanitized
# one from build.py --sanitize); by default the in-tree libmoe.so.
LIB_PATH = os.environ.get("MOE_LIB") or os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EHIP, MOE_EFULL = 0, -1, -2, -3, -4
MOE_RES_LO, MOE_RES_PROMOTING, MOE_RES_HI, MOE_RES_EVICTING = 0, 1, 2, 3
MOE_RES_FORCE_UPDATE, MOE_RES_WAIT = 1, 2
MOE_ROUTE_TOPK, MOE_ROUTE_OEA, MOE_ROUTE_PRUNED = 0, 1, 2
MOE_DT_F32, MOE_DT_BF16 = 0, 1
MOE_W_F32, MOE_W_BF16, MOE_W_INT4_G128 = 0, 1, 2


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


class ExpertHandle(ctypes.Structure):
    """Mirror of moe_expert_handle (64 bytes)."""
    _fields_ = [("fmt", ctypes.c_int32), ("group", ctypes.c_int32),
                ("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
                ("s_gate", ctypes.c_void_p), ("s_up", ctypes.c_void_p), ("s_down", ctypes.c_void_p),
                ("reserved", ctypes.c_int64)]


HANDLE_BYTES = ctypes.sizeof(ExpertHandle)
assert HANDLE_BYTES == 64


class ResidencyConfig(ctypes.Structure):
    """Mirror of moe_residency_config (include/moe_residency.h)."""
    _fields_ = [("N", ctypes.c_int), ("H", ctypes.c_int), ("I", ctypes.c_int),
                ("table", ctypes.c_void_p), ("lo", ctypes.POINTER(ExpertHandle)),
                ("hi_src", ctypes.POINTER(ctypes.c_void_p)), ("pool_hi", ctypes.c_void_p),
                ("budget", ctypes.c_void_p), ("S", ctypes.c_void_p), ("c", ctypes.c_void_p),
                ("S_host", ctypes.c_void_p), ("n_hi", ctypes.c_int), ("alpha", ctypes.c_float),
                ("margin", ctypes.c_float), ("interval_s", ctypes.c_double),
                ("compute_stream", ctypes.c_void_p), ("mig_stream", ctypes.c_void_p)]


class ResidencyStats(ctypes.Structure):
    """Mirror of moe_residency_stats."""
    _fields_ = [(n, ctypes.c_int64) for n in (
        "steps", "updates", "decisions", "promotions_started", "promotions_published", "demotions",
        "evictions", "deferred", "bytes_h2d")]

    def as_dict(self) -> dict:
        return {n: getattr(self, n) for n, _ in self._fields_}

_lib = None

# (name, argtypes, restype)
_P, _I, _F, _S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_SIGNATURES = [
    ("moe_router_logits", [_P, _I, _P, _I, _I, _I, _P, _P], _I),
    ("moe_route_topk", [_P, _I, _I, _I, _I, _P, _P, _P], _I),
    ("moe_route_oea", [_P, _I, _I, _I, _F, _I, _P, _P, _P, _P, _P, _P], _I),
    ("moe_dispatch", [_P, _I, _I, _I, _P, _P, _P, _P, _P, _P], _I),
    ("moe_route_dispatch", [_P, _I, _I, _I, _I, _I, _F, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
     _I),
    ("moe_router_route_dispatch", [_P, _I, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I] + [_P] * 14, _I),
    ("moe_ffn_workspace_bytes", [_I, _I, _I, _I], _S),
    ("moe_expert_ffn", [_P, _I, _I, _I, _P, _I, _P, _P, _P, _P, _P, _P, _I, _I, _P, _P, _S, _P], _I),
    ("moe_expert_ffn_noalloc", [_P, _I, _I, _I, _P, _I, _P, _P, _P, _P, _P, _P, _I, _I, _P, _P], _I),
    ("moe_handle_publish", [_P, _I, ctypes.POINTER(ExpertHandle), _P], _I),
    ("moe_quantize_int4_g128", [_P, _I, _I, _P, _P, _P], _I),
    ("moe_pack_weights", [_I, _P, _P, _I, _I, _P, _P, _P], _I),
    ("moe_hotness_ema", [_P, _P, _I, _F, _P], _I),
    ("moe_pool_create", [_P, _S, _S, ctypes.POINTER(_P)], _I),
    ("moe_pool_destroy", [_P], None),
    ("moe_pool_alloc", [_P, ctypes.POINTER(_P)], _I),
    ("moe_pool_free", [_P, _P], _I),
    ("moe_pool_free_blocks", [_P], _I),
    ("moe_pool_total_blocks", [_P], _I),
    ("moe_pool_block_bytes", [_P], _S),
    ("moe_budget_create", [_S, _S, ctypes.POINTER(_P)], _I),
    ("moe_budget_destroy", [_P], None),
    ("moe_budget_try_reserve", [_P, _S], _I),
    ("moe_budget_release", [_P, _S], _I),
    ("moe_budget_used", [_P], _S),
    ("moe_budget_capacity", [_P], _S),
    ("moe_residency_select", [_P, _P, _P, _I, _I, _F, _P, _P, ctypes.POINTER(_I), _P, ctypes.POINTER(_I)], _I),
    ("moe_residency_create", [ctypes.POINTER(ResidencyConfig), ctypes.POINTER(_P)], _I),
    ("moe_residency_step", [_P, _P, _I], _I),
    ("moe_residency_state", [_P, _I], _I),
    ("moe_residency_pending", [_P], _I),
    ("moe_residency_get_stats", [_P, ctypes.POINTER(ResidencyStats)], _I),
    ("moe_residency_destroy", [_P], _I),
    ("moe_stream_read", [_P, _S, _I, _P, _P], _I),
    ("moe_expert_ffn_phase_events", [_P, _I, _I, _I, _P, _I, _P, _P, _P, _P, _P, _P, _I, _I, _P, _P, _S, _P, _P],
     _I),
    ("moe_status_str", [_I], ctypes.c_char_p),
    ("moe_last_error", [], ctypes.c_char_p),
]
EXPORTED = [name for name, _, _ in _SIGNATURES]


def lib():
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libmoe.so not found at {LIB_PATH}; build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`")
    l = ctypes.CDLL(LIB_PATH)
    for name, args, res in _SIGNATURES:
        f = getattr(l, name)
        f.argtypes = args
        f.restype = res
    _lib = l
    return l


def _check(fn: str, status: int):
    if status != MOE_OK:
        raise MoeError(fn, status, lib().moe_last_error().decode())


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmoe must be contiguous")
    return t.data_ptr()


def _check_i32_table(t, need: int, name: str, device) -> None:
    """A device int32 table the kernels index on the device (n_valid[0],
    k0_by_batch[b] for b <= B): wrong placement, type or length would be an
    out-of-bounds device read, so it is refused here."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or t.device != device:
        raise ValueError(f"{name} must be an int32 tensor on {device}")
    if not t.is_contiguous() or t.numel() < need:
        raise ValueError(f"{name} must be contiguous with at least {need} entries (has {t.numel()})")


def _stream(stream=None) -> int:
    """The raw HIP stream handle to launch on: `stream`'s (a torch stream or
    an int handle), else the current stream of the current device (read
    without building a torch Stream object, which costs microseconds per call)."""
    if stream is None:
        return torch._C._cuda_getCurrentRawStream(torch.cuda.current_device())
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _x_dtype(x: torch.Tensor) -> int:
    if x.dtype == torch.bfloat16:
        return MOE_DT_BF16
    if x.dtype == torch.float32:
        return MOE_DT_F32
    raise TypeError(f"activations must be float32 or bfloat16, got {x.dtype}")


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI, minus the moe_ prefix)
# ---------------------------------------------------------------------------
def router_logits(x, w_r, logits=None, stream=None):
    B, H = x.shape
    N = w_r.shape[0]
    if logits is None:
        logits = torch.empty(B, N, device=x.device, dtype=torch.float32)
    _check("moe_router_logits", lib().moe_router_logits(_ptr(x), _x_dtype(x), _ptr(w_r), B, H, N,
                                                        _ptr(logits), _stream(stream)))
    return logits


def route_topk(logits, k: int, renorm: bool = True, idx=None, w=None, stream=None):
    B, N = logits.shape
    dev = logits.device
    idx = torch.empty(B, k, device=dev, dtype=torch.int32) if idx is None else idx
    w = torch.empty(B, k, device=dev, dtype=torch.float32) if w is None else w
    _check("moe_route_topk", lib().moe_route_topk(_ptr(logits), B, N, k, int(bool(renorm)), _ptr(idx),
                                                  _ptr(w), _stream(stream)))
    return idx, w


def route_oea(logits, k0: int, p: float, k: int, out=None, stream=None):
    """Returns dict idx, w, n_base, mask, T (device tensors)."""
    B, N = logits.shape
    dev = logits.device
    if out is None:
        out = dict(idx=torch.empty(B, k, device=dev, dtype=torch.int32),
                   w=torch.empty(B, k, device=dev, dtype=torch.float32),
                   n_base=torch.empty(B, device=dev, dtype=torch.int32),
                   mask=torch.empty((N + 31) // 32, device=dev, dtype=torch.int32),
                   T=torch.empty(1, device=dev, dtype=torch.int32))
    _check("moe_route_oea", lib().moe_route_oea(_ptr(logits), B, N, k0, float(p), k, _ptr(out["idx"]),
                                                _ptr(out["w"]), _ptr(out.get("n_base")),
                                                _ptr(out.get("mask")), _ptr(out.get("T")),
                                                _stream(stream)))
    return out


def dispatch(idx, N: int, out=None, stream=None):
    """Returns dict cnt, offsets, perm, active, T (device tensors)."""
    B, k = idx.shape
    dev = idx.device
    if out is None:
        out = dict(cnt=torch.empty(N, device=dev, dtype=torch.int32),
                   offsets=torch.empty(N + 1, device=dev, dtype=torch.int32),
                   perm=torch.empty(B * k, device=dev, dtype=torch.int32),
                   active=torch.empty(N, device=dev, dtype=torch.int32),
                   T=torch.empty(1, device=dev, dtype=torch.int32))
    _check("moe_dispatch", lib().moe_dispatch(_ptr(idx), B, N, k, _ptr(out["cnt"]), _ptr(out["offsets"]),
                                              _ptr(out["perm"]), _ptr(out["active"]), _ptr(out["T"]),
                                              _stream(stream)))
    return out


def route_dispatch(logits, k: int, mode: str, k0: int = 0, p: float = 1.0, renorm: bool = True,
                   route=None, disp=None, stream=None, max_p: int | None = None, n_valid=None,
                   k0_by_batch=None, sync=None):
    """Routing ("topk", "oea" or "pruned") and dispatch (one launch up to 48 tokens).

    max_p: OEA Phase 2 rank limit (default N); n_valid: optional device int32
    tensor [1] with the number of real tokens; k0_by_batch: optional device
    int32 tensor [B+1], the k0 to use for each real batch size; sync: optional
    device int32 [1], zero on entry and left at zero (vanilla top-k above 48
    tokens then dispatches in its routing launch).  Returns (route, disp)
    dicts.
    """
    B, N = logits.shape
    dev = logits.device
    i32 = dict(device=dev, dtype=torch.int32)
    if route is None:
        route = dict(idx=torch.empty(B, k, **i32), w=torch.empty(B, k, device=dev, dtype=torch.float32),
                     n_base=torch.empty(B, **i32), mask=torch.empty((N + 31) // 32, **i32))
    if disp is None:
        disp = dict(cnt=torch.empty(N, **i32), offsets=torch.empty(N + 1, **i32), perm=torch.empty(B * k, **i32),
                    active=torch.empty(N, **i32), T=torch.empty(1, **i32))
    m = {"topk": MOE_ROUTE_TOPK, "oea": MOE_ROUTE_OEA, "pruned": MOE_ROUTE_PRUNED}[mode]
    _check_i32_table(n_valid, 1, "n_valid", dev)
    _check_i32_table(k0_by_batch, B + 1, "k0_by_batch", dev)
    _check_i32_table(sync, 1, "sync", dev)
    _check("moe_route_dispatch", lib().moe_route_dispatch(
        _ptr(logits), B, N, k, m, int(k0), float(p), N if max_p is None else int(max_p), int(bool(renorm)),
        _ptr(n_valid), _ptr(k0_by_batch), _ptr(route["idx"]), _ptr(route["w"]), _ptr(route.get("n_base")), _ptr(route.get("mask")),
        _ptr(disp["cnt"]), _ptr(disp["offsets"]), _ptr(disp["perm"]), _ptr(disp["active"]), _ptr(disp["T"]),
        _ptr(sync), _stream(stream)))
    return route, disp


def router_route_dispatch(x, w_r, k: int, mode: str, k0: int = 0, p: float = 1.0, renorm: bool = True,
                          route=None, disp=None, logits=None, sync=None, stream=None, max_p: int | None = None,
                          n_valid=None, k0_by_batch=None):
    """Router logits, routing and dispatch (one launch up to 48 tokens).  sync: device int32
    [1] that starts at zero (allocated here if None).  Returns (logits, route,
    disp)."""
    B, H = x.shape
    N = w_r.shape[0]
    dev = x.device
    i32 = dict(device=dev, dtype=torch.int32)
    logits = torch.empty(B, N, device=dev, dtype=torch.float32) if logits is None else logits
    sync = torch.zeros(1, **i32) if sync is None else sync
    if route is None:
        route = dict(idx=torch.empty(B, k, **i32), w=torch.empty(B, k, device=dev, dtype=torch.float32),
                     n_base=torch.empty(B, **i32), mask=torch.empty((N + 31) // 32, **i32))
    if disp is None:
        disp = dict(cnt=torch.empty(N, **i32), offsets=torch.empty(N + 1, **i32), perm=torch.empty(B * k, **i32),
                    active=torch.empty(N, **i32), T=torch.empty(1, **i32))
    m = {"topk": MOE_ROUTE_TOPK, "oea": MOE_ROUTE_OEA, "pruned": MOE_ROUTE_PRUNED}[mode]
    _check_i32_table(n_valid, 1, "n_valid", dev)
    _check_i32_table(k0_by_batch, B + 1, "k0_by_batch", dev)
    _check_i32_table(sync, 1, "sync", dev)
    _check("moe_router_route_dispatch", lib().moe_router_route_dispatch(
        _ptr(x), _x_dtype(x), _ptr(w_r), B, H, N, k, m, int(k0), float(p), N if max_p is None else int(max_p),
        int(bool(renorm)), _ptr(n_valid), _ptr(k0_by_batch), _ptr(logits), _ptr(route["idx"]), _ptr(route["w"]),
        _ptr(route.get("n_base")), _ptr(route.get("mask")), _ptr(disp["cnt"]), _ptr(disp["offsets"]),
        _ptr(disp["perm"]), _ptr(disp["active"]), _ptr(disp["T"]), _ptr(sync), _stream(stream)))
    return logits, route, disp


def ffn_workspace_bytes(B: int, k: int, H: int, I: int) -> int:
    return int(lib().moe_ffn_workspace_bytes(B, k, H, I))


def expert_ffn(table, N: int, H: int, I: int, x, idx, w, disp, y=None, ws=None, stream=None):
    B, k = idx.shape
    dev = x.device
    if y is None:
        y = torch.empty(B, H, device=dev, dtype=torch.float32)
    if ws is None:   # (a caller's workspace is checked for size by the library)
        ws = torch.zeros(ffn_workspace_bytes(B, k, H, I), device=dev, dtype=torch.uint8)
    _check("moe_expert_ffn", lib().moe_expert_ffn(
        _ptr(table), N, H, I, _ptr(x), _x_dtype(x), _ptr(idx), _ptr(w), _ptr(disp["offsets"]),
        _ptr(disp["perm"]), _ptr(disp["active"]), _ptr(disp["T"]), B, k, _ptr(y), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))
    return y


NOALLOC_WORKSPACE_BYTES = 32 << 20   # MOE_FFN_NOALLOC_WORKSPACE_BYTES


def expert_ffn_noalloc(table, N: int, H: int, I: int, x, idx, w, disp, y, stream=None):
    """moe_expert_ffn_noalloc: the expert FFN with the library's static
    workspace (the caller passes inputs and the output y only)."""
    B, k = idx.shape
    _check("moe_expert_ffn_noalloc", lib().moe_expert_ffn_noalloc(
        _ptr(table), N, H, I, _ptr(x), _x_dtype(x), _ptr(idx), _ptr(w), _ptr(disp["offsets"]),
        _ptr(disp["perm"]), _ptr(disp["active"]), _ptr(disp["T"]), B, k, _ptr(y), _stream(stream)))
    return y


def handle_publish(table, e: int, h: ExpertHandle, stream=None):
    _check("moe_handle_publish", lib().moe_handle_publish(_ptr(table), e, ctypes.byref(h), _stream(stream)))


def quantize_int4_g128(w_bf16, q=None, scales=None, stream=None):
    rows, cols = w_bf16.shape
    dev = w_bf16.device
    q = torch.empty(rows, cols // 2, device=dev, dtype=torch.uint8) if q is None else q
    scales = torch.empty(rows, cols // 128, device=dev, dtype=torch.int16) if scales is None else scales
    _check("moe_quantize_int4_g128", lib().moe_quantize_int4_g128(_ptr(w_bf16), rows, cols, _ptr(q),
                                                                  _ptr(scales), _stream(stream)))
    return q, scales


def pack_weights(fmt: int, src, scales=None, dst=None, dst_scales=None, stream=None):
    """Pack a row-major [rows, cols] matrix (INT4: the quantiser's bytes and
    scales) into the tiled layout the expert FFN reads."""
    rows = src.shape[0]
    cols = {MOE_W_F32: src.shape[1], MOE_W_BF16: src.shape[1], MOE_W_INT4_G128: src.shape[1] * 2}[fmt]
    dst = torch.empty_like(src) if dst is None else dst
    if fmt == MOE_W_INT4_G128 and dst_scales is None:
        dst_scales = torch.empty_like(scales)
    _check("moe_pack_weights", lib().moe_pack_weights(fmt, _ptr(src), _ptr(scales), rows, cols, _ptr(dst),
                                                      _ptr(dst_scales), _stream(stream)))
    return dst, dst_scales


def hotness_ema(S, cnt, alpha: float, stream=None):
    _check("moe_hotness_ema", lib().moe_hotness_ema(_ptr(S), _ptr(cnt), S.shape[0], float(alpha),
                                                    _stream(stream)))
    return S


def stream_read(buf, out, waves_per_cu: int = 8, stream=None):
    """moe_stream_read: one read pass over buf (the HBM read-ceiling probe);
    XORs buf's 32-bit words into out[0]."""
    _check("moe_stream_read", lib().moe_stream_read(_ptr(buf), buf.numel() * buf.element_size(), int(waves_per_cu),
                                                    _ptr(out), _stream(stream)))
    return out


def expert_ffn_phase_events(table, N: int, H: int, I: int, x, idx, w, disp, y, ws, events, stream=None):
    """moe_expert_ffn_phase_events: the expert FFN call with four torch.cuda
    Events (timing enabled) recorded before phase A, after phase A, after
    phase B and after the combine, on the stream the kernels run on."""
    if len(events) != 4:
        raise ValueError("four events")
    st = stream if stream is not None else torch.cuda.current_stream()
    handles = (ctypes.c_void_p * 4)()
    for i, ev in enumerate(events):
        if ev.cuda_event == 0:   # torch creates the HIP event on its first record
            ev.record(st)
        handles[i] = ev.cuda_event
    B, k = idx.shape
    _check("moe_expert_ffn_phase_events", lib().moe_expert_ffn_phase_events(
        _ptr(table), N, H, I, _ptr(x), _x_dtype(x), _ptr(idx), _ptr(w), _ptr(disp["offsets"]),
        _ptr(disp["perm"]), _ptr(disp["active"]), _ptr(disp["T"]), B, k, _ptr(y), _ptr(ws),
        ws.numel() * ws.element_size(), ctypes.cast(handles, ctypes.c_void_p), _stream(stream)))
    return y


def status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


# ---------------------------------------------------------------------------
# residency (include/moe_residency.h): host objects behind opaque pointers
# ---------------------------------------------------------------------------
def pool_create(arena_ptr: int, arena_bytes: int, block_bytes: int) -> int:
    out = ctypes.c_void_p()
    _check("moe_pool_create", lib().moe_pool_create(arena_ptr, arena_bytes, block_bytes, ctypes.byref(out)))
    return out.value


def pool_alloc(pool: int) -> int | None:
    blk = ctypes.c_void_p()
    st = lib().moe_pool_alloc(pool, ctypes.byref(blk))
    if st == MOE_EFULL:
        return None
    _check("moe_pool_alloc", st)
    return blk.value


def pool_free(pool: int, block: int):
    _check("moe_pool_free", lib().moe_pool_free(pool, block))


def budget_create(total: int, fixed: int) -> int:
    out = ctypes.c_void_p()
    _check("moe_budget_create", lib().moe_budget_create(total, fixed, ctypes.byref(out)))
    return out.value


def budget_try_reserve(budget: int, nbytes: int) -> bool:
    st = lib().moe_budget_try_reserve(budget, nbytes)
    if st < 0:
        _check("moe_budget_try_reserve", st)
    return st == 1


def budget_release(budget: int, nbytes: int):
    _check("moe_budget_release", lib().moe_budget_release(budget, nbytes))


def residency_select(S, in_hi, n_hi: int, margin: float, locked=None):
    """Host policy update on numpy arrays: returns (target, promote, demote)."""
    import numpy as np
    S = np.ascontiguousarray(S, dtype=np.float32)
    N = S.shape[0]
    in_hi = np.ascontiguousarray(in_hi, dtype=np.uint8)
    lk = None if locked is None else np.ascontiguousarray(locked, dtype=np.uint8)
    target = np.zeros(N, np.uint8)
    pro = np.zeros(N, np.int32)
    dem = np.zeros(N, np.int32)
    npro, ndem = ctypes.c_int(), ctypes.c_int()
    _check("moe_residency_select", lib().moe_residency_select(
        S.ctypes.data, in_hi.ctypes.data, None if lk is None else lk.ctypes.data, N, n_hi, float(margin),
        target.ctypes.data, pro.ctypes.data, ctypes.byref(npro), dem.ctypes.data, ctypes.byref(ndem)))
    return target.astype(bool), pro[:npro.value].tolist(), dem[:ndem.value].tolist()


def residency_create(cfg: ResidencyConfig) -> int:
    out = ctypes.c_void_p()
    _check("moe_residency_create", lib().moe_residency_create(ctypes.byref(cfg), ctypes.byref(out)))
    return out.value


def residency_step(res: int, cnt=None, force: bool = False, wait: bool = False):
    flags = (MOE_RES_FORCE_UPDATE if force else 0) | (MOE_RES_WAIT if wait else 0)
    _check("moe_residency_step", lib().moe_residency_step(res, _ptr(cnt), flags))


def residency_stats(res: int) -> dict:
    st = ResidencyStats()
    _check("moe_residency_get_stats", lib().moe_residency_get_stats(res, ctypes.byref(st)))
    return st.as_dict()
