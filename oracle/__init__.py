"""CPU oracle for the decode MoE layer with OEA routing -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The GPU library never does, and this package never imports the
GPU library: the two share no code.

The arithmetic lives in ``moe_oracle.c`` (plain C, fp64 accumulation); this
module only marshals numpy arrays through ctypes.  Page and section citations
for every step are in the C file's comments.

Parity status: every function is pinned by ``tests/test_oracle_pins.py``
(closed forms, brute force, library special cases).  The expert FFN has no
worked example on the pages, so it is pinned only through invariants that hold
for any correct SwiGLU MoE layer (identical experts reduce to a dense MLP whose
value numpy computes, scaled down-projections scale the output, zero up
projections give zero).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_BUILD = os.path.join(_HERE, "_build")
# MOE_ORACLE_LIB selects the sanitized build (build(sanitize=True))
_LIB_PATH = os.environ.get("MOE_ORACLE_LIB") or os.path.join(_BUILD, "libmoe_oracle.so")
ASAN_LIB_PATH = os.path.join(_BUILD, "asan", "libmoe_oracle.so")

_lib = None


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile the oracle with gcc (plain -O2, IEEE arithmetic, no contraction).
    sanitize=True: the same flags with AddressSanitizer and
    UndefinedBehaviorSanitizer, built with ROCm's clang (whose sanitizer
    runtime the sanitized libmoe uses too), into _build/asan/."""
    path = ASAN_LIB_PATH if sanitize else _LIB_PATH
    if not force and os.path.exists(path):
        return path
    os.makedirs(os.path.dirname(path), exist_ok=True)
    tmp = path + ".tmp%d" % os.getpid()
    if sanitize:
        cmd = ["/opt/rocm/llvm/bin/clang", "-O1", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-fopenmp", "-Wall", "-fsanitize=address,undefined",
               "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-o", tmp, _SRC, "-lm"]
    else:
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-fopenmp", "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, path)
    return path


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.environ.get("MOE_ORACLE_LIB") and (not os.path.exists(_LIB_PATH) or
                                                 os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.orc_cexpf.argtypes = [ctypes.c_float]
    lib.orc_cexpf.restype = ctypes.c_float
    lib.orc_f32_to_f16.argtypes = [ctypes.c_float]
    lib.orc_f32_to_f16.restype = ctypes.c_uint16
    lib.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
    lib.orc_f16_to_f32.restype = ctypes.c_float
    lib.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_to_f32.restype = ctypes.c_float
    lib.orc_rank.argtypes = [P, I, P]
    lib.orc_softmax_terms.argtypes = [P, I, P, P]
    lib.orc_topp_count.argtypes = [P, ctypes.c_float, P, I, ctypes.c_float]
    lib.orc_topp_count.restype = I
    lib.orc_route.argtypes = [P, I, I, I, I, ctypes.c_float, I, I, P, P, P, P, P]
    lib.orc_route_general.argtypes = [P, I, I, I, I, ctypes.c_float, I, I, I, I, P, P, P, P, P]
    lib.orc_dispatch.argtypes = [P, I, I, I, P, P, P, P, P]
    lib.orc_router_logits.argtypes = [P, P, I, I, I, P]
    lib.orc_expert_ffn.argtypes = [P, I, I, P, P, P, I, I, P]
    lib.orc_quantize_int4.argtypes = [P, I, I, P, P]
    lib.orc_hotness_ema.argtypes = [P, P, I, ctypes.c_double]
    lib.orc_set_threads.argtypes = [I]
    lib.orc_get_threads.restype = I
    lib.orc_set_threads(_default_threads())
    _lib = lib
    return lib


def _default_threads() -> int:
    """OMP_NUM_THREADS if set, else the usable cores, at most 16."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def set_threads(n: int) -> None:
    """Threads of the expert FFN's OpenMP loops (results do not depend on it)."""
    _load().orc_set_threads(int(n))


def get_threads() -> int:
    return int(_load().orc_get_threads())


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# --------------------------------------------------------------------------
# scalar helpers
# --------------------------------------------------------------------------
def cexpf(x: float) -> float:
    return float(_load().orc_cexpf(ctypes.c_float(x)))


def f32_to_f16(x: float) -> int:
    return int(_load().orc_f32_to_f16(ctypes.c_float(x)))


def f16_to_f32(h: int) -> float:
    return float(_load().orc_f16_to_f32(ctypes.c_uint16(h)))


def bf16_to_f32(b: int) -> float:
    return float(_load().orc_bf16_to_f32(ctypes.c_uint16(b)))


# --------------------------------------------------------------------------
# routing
# --------------------------------------------------------------------------
def rank(logits_row) -> np.ndarray:
    l = _c(logits_row, np.float32)
    out = np.zeros(l.shape[0], np.int32)
    _load().orc_rank(_ptr(l), l.shape[0], _ptr(out))
    return out


def softmax_terms(logits_row):
    l = _c(logits_row, np.float32)
    e = np.zeros(l.shape[0], np.float32)
    Z = np.zeros(1, np.float32)
    _load().orc_softmax_terms(_ptr(l), l.shape[0], _ptr(e), _ptr(Z))
    return e, float(Z[0])


def topp_count(logits_row, p: float) -> int:
    l = _c(logits_row, np.float32)
    e, Z = softmax_terms(l)
    order = rank(l)
    return int(_load().orc_topp_count(_ptr(e), ctypes.c_float(Z), _ptr(order), l.shape[0],
                                      ctypes.c_float(p)))


def route(logits, k: int, *, oea: bool, k0: int = 0, p: float = 1.0, renorm: bool = True,
          pruned: bool = False, max_p: int | None = None, n_valid: int | None = None):
    """Vanilla top-k (oea=False) or OEA (oea=True) routing of fp32 logits [B, N].

    pruned=True keeps only OEA's Phase 1 baseline; max_p limits Phase 2 to
    the token's ranks up to max_p (default N); k is the slot count (the
    page's k_max for OEA); tokens i >= n_valid (default B) are padding.
    Returns a dict: idx [B,k] int32 (-1 pad), w [B,k] float64 (0 pad),
    n_base [B] int32, mask [ceil(N/32)] uint32, T int.
    """
    l = _c(logits, np.float32)
    B, N = l.shape
    idx = np.zeros((B, k), np.int32)
    w = np.zeros((B, k), np.float64)
    n_base = np.zeros(B, np.int32)
    mask = np.zeros((N + 31) // 32, np.uint32)
    T = np.zeros(1, np.int32)
    mode = 0 if not oea else (2 if pruned else 1)
    _load().orc_route_general(_ptr(l), B, N, k, k0, ctypes.c_float(p), mode, N if max_p is None else int(max_p),
                              int(renorm), B if n_valid is None else int(n_valid),
                              _ptr(idx), _ptr(w), _ptr(n_base), _ptr(mask), _ptr(T))
    return {"idx": idx, "w": w, "n_base": n_base, "mask": mask, "T": int(T[0])}


def dispatch(idx, N: int):
    idx = _c(idx, np.int32)
    B, k = idx.shape
    cnt = np.zeros(N, np.int32)
    offsets = np.zeros(N + 1, np.int32)
    perm = np.zeros(B * k, np.int32)
    active = np.zeros(N, np.int32)
    T = np.zeros(1, np.int32)
    _load().orc_dispatch(_ptr(idx), B, N, k, _ptr(cnt), _ptr(offsets), _ptr(perm), _ptr(active),
                         _ptr(T))
    return {"cnt": cnt, "offsets": offsets, "perm": perm, "active": active, "T": int(T[0])}


def router_logits(x, wr) -> np.ndarray:
    """x [B,H] and W_r [N,H] widened to float64; returns float64 logits [B,N]."""
    x = _c(x, np.float64)
    wr = _c(wr, np.float64)
    B, H = x.shape
    N = wr.shape[0]
    out = np.zeros((B, N), np.float64)
    _load().orc_router_logits(_ptr(x), _ptr(wr), B, H, N, _ptr(out))
    return out


# --------------------------------------------------------------------------
# expert FFN
# --------------------------------------------------------------------------
FMT_F32, FMT_BF16, FMT_INT4 = 0, 1, 2


class _Expert(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("pad", ctypes.c_int32),
                ("gate", ctypes.c_void_p), ("up", ctypes.c_void_p), ("down", ctypes.c_void_p),
                ("s_gate", ctypes.c_void_p), ("s_up", ctypes.c_void_p), ("s_down", ctypes.c_void_p)]


def expert_ffn(experts, H: int, I: int, x, idx, w) -> np.ndarray:
    """SwiGLU experts + weighted combine in double.

    experts: list of dicts with 'fmt' and arrays 'gate' [I,H], 'up' [I,H], 'down' [H,I]
             (float32 for FMT_F32, uint16 bf16 bits for FMT_BF16, packed uint8 for
             FMT_INT4 with 's_gate','s_up','s_down' uint16 fp16 scales).
    x: [B,H] values (widened exactly), idx [B,k] int32, w [B,k] float64.
    """
    x = _c(x, np.float64)
    idx = _c(idx, np.int32)
    w = _c(w, np.float64)
    B, k = idx.shape
    keep = []
    arr = (_Expert * len(experts))()
    for e, ex in enumerate(experts):
        fmt = int(ex["fmt"])
        dt = {FMT_F32: np.float32, FMT_BF16: np.uint16, FMT_INT4: np.uint8}[fmt]
        mats = [_c(ex[n], dt) for n in ("gate", "up", "down")]
        keep += mats
        arr[e].fmt = fmt
        arr[e].gate, arr[e].up, arr[e].down = [m.ctypes.data for m in mats]
        if fmt == FMT_INT4:
            sc = [_c(ex[n], np.uint16) for n in ("s_gate", "s_up", "s_down")]
            keep += sc
            arr[e].s_gate, arr[e].s_up, arr[e].s_down = [s.ctypes.data for s in sc]
    y = np.zeros((B, H), np.float64)
    _load().orc_expert_ffn(ctypes.cast(arr, ctypes.c_void_p), H, I, _ptr(x), _ptr(idx), _ptr(w),
                           B, k, _ptr(y))
    del keep
    return y


def quantize_int4(w_bf16_bits):
    """[rows, cols] bf16 bits -> (packed uint8 [rows, cols/2], fp16 scale bits [rows, cols/128])."""
    wb = _c(w_bf16_bits, np.uint16)
    rows, cols = wb.shape
    if cols % 128:
        raise ValueError("cols must be a multiple of 128")
    q = np.zeros((rows, cols // 2), np.uint8)
    s = np.zeros((rows, cols // 128), np.uint16)
    _load().orc_quantize_int4(_ptr(wb), rows, cols, _ptr(q), _ptr(s))
    return q, s


def hotness_ema(S, counts, alpha: float) -> np.ndarray:
    S = np.array(S, np.float64, copy=True)
    c = _c(counts, np.int32)
    _load().orc_hotness_ema(_ptr(S), _ptr(c), S.shape[0], ctypes.c_double(alpha))
    return S
