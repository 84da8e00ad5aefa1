"""CPU-only checks of the C ABI: the library loads, exports every entry point
include/moe.h declares, and rejects invalid arguments on the host before
anything is launched (no call here reaches a kernel)."""
import ctypes
import os
import re

import pytest

import aware_expert_routing_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

FAKE = ctypes.c_void_p(1 << 20)   # never dereferenced: every call below fails validation


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert set(_declared()) == set(moe.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = moe.lib()
    for name in _declared():
        assert hasattr(lib, name), name


def test_handle_record_is_64_bytes():
    assert ctypes.sizeof(moe.ExpertHandle) == moe.HANDLE_BYTES == 64


def test_status_strings():
    assert moe.status_str(0) == "ok"
    assert moe.status_str(-1) == "invalid argument"
    assert moe.status_str(-2) == "unsupported size"
    assert moe.status_str(-3) == "HIP runtime error"


def test_workspace_size():
    assert moe.ffn_workspace_bytes(16, 8, 2048, 768) == 16 * 8 * (2048 + 768) * 4
    assert moe.ffn_workspace_bytes(0, 8, 2048, 768) == 0


@pytest.mark.parametrize("B,N,k,status", [
    (16, 0, 1, -1), (16, 129, 8, -1), (16, 8, 9, -1), (16, 128, 17, -1), (16, 128, 0, -1),
    (0, 128, 8, -1), (129, 128, 8, -2),
])
def test_route_topk_rejects_sizes(B, N, k, status):
    lib = moe.lib()
    assert lib.moe_route_topk(FAKE, B, N, k, 1, FAKE, FAKE, None) == status


@pytest.mark.parametrize("k0,p,k", [(0, 1.0, 8), (9, 1.0, 8), (3, 0.0, 8), (3, -0.5, 8), (3, float("nan"), 8)])
def test_route_oea_rejects_knobs(k0, p, k):
    lib = moe.lib()
    assert lib.moe_route_oea(FAKE, 16, 128, k0, p, k, FAKE, FAKE, None, None, None, None) == -1
    assert "k0" in lib.moe_last_error().decode() or "p must" in lib.moe_last_error().decode()


def test_null_pointers_rejected():
    lib = moe.lib()
    assert lib.moe_route_topk(None, 4, 16, 4, 1, FAKE, FAKE, None) == -1
    assert lib.moe_route_oea(FAKE, 4, 16, 2, 0.7, 4, None, FAKE, None, None, None, None) == -1
    assert lib.moe_dispatch(FAKE, 4, 16, 4, FAKE, FAKE, FAKE, None, FAKE, None) == -1
    assert lib.moe_router_logits(None, 0, FAKE, 4, 256, 16, FAKE, None) == -1
    assert lib.moe_quantize_int4_g128(FAKE, 4, 256, None, FAKE, None) == -1
    assert lib.moe_hotness_ema(None, FAKE, 16, 0.9, None) == -1
    assert lib.moe_handle_publish(None, 0, None, None) == -1


def test_expert_ffn_rejects_bad_shapes_and_small_workspace():
    lib = moe.lib()
    args = lambda H, I, ws: (FAKE, 128, H, I, FAKE, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, 8, FAKE,
                             FAKE, ws, None)
    need = moe.ffn_workspace_bytes(16, 8, 2048, 768)
    assert lib.moe_expert_ffn(*args(2046, 768, need)) == -1          # H % 8
    assert lib.moe_expert_ffn(*args(2048, 770, need)) == -1          # I % 8
    assert lib.moe_expert_ffn(*args(2048, 768, need - 1)) == -1      # workspace
    assert lib.moe_expert_ffn(*args(32768, 768, 1 << 40)) == -2      # beyond limits
    bad_dtype = list(args(2048, 768, need))
    bad_dtype[5] = 7
    assert lib.moe_expert_ffn(*bad_dtype) == -1


def test_router_logits_rejects_bad_hidden():
    lib = moe.lib()
    assert lib.moe_router_logits(FAKE, 1, FAKE, 4, 250, 16, FAKE, None) == -1
    assert lib.moe_router_logits(FAKE, 3, FAKE, 4, 256, 16, FAKE, None) == -1
    assert lib.moe_router_logits(FAKE, 1, FAKE, 200, 256, 16, FAKE, None) == -2


def test_publish_rejects_bad_handles():
    lib = moe.lib()
    h = moe.ExpertHandle()
    h.fmt = 5
    assert lib.moe_handle_publish(FAKE, 0, ctypes.byref(h), None) == -1
    h.fmt = moe.MOE_W_INT4_G128
    h.w_gate = h.w_up = h.w_down = 1 << 20
    h.group = 64
    assert lib.moe_handle_publish(FAKE, 0, ctypes.byref(h), None) == -1
    h.fmt = moe.MOE_W_BF16
    assert lib.moe_handle_publish(FAKE, 128, ctypes.byref(h), None) == -1


def test_quantizer_rejects_ragged_groups():
    lib = moe.lib()
    assert lib.moe_quantize_int4_g128(FAKE, 4, 200, FAKE, FAKE, None) == -1


def test_pack_rejects_bad_arguments():
    lib = moe.lib()
    dst = ctypes.c_void_p(1 << 30)
    ok = (moe.MOE_W_BF16, FAKE, None, 32, 64, dst, None, None)

    def call(**kw):
        names = ["fmt", "src", "src_scales", "rows", "cols", "dst", "dst_scales", "stream"]
        args = dict(zip(names, ok))
        args.update(kw)
        return lib.moe_pack_weights(*[args[n] for n in names])

    assert call(fmt=7) == -1
    assert call(src=None) == -1
    assert call(rows=24) == -1                                   # rows % 16
    assert call(cols=48) == -1                                   # bf16 needs cols % 32
    assert call(fmt=moe.MOE_W_F32, cols=40) == -1                # fp32 needs cols % 16
    assert call(fmt=moe.MOE_W_INT4_G128, cols=128) == -1         # INT4 needs scale pointers
    assert call(fmt=moe.MOE_W_INT4_G128, cols=64, src_scales=FAKE, dst_scales=dst) == -1
    assert call(src=ctypes.c_void_p((1 << 20) + 8)) == -1       # 16-byte alignment
    assert call(dst=ctypes.c_void_p((1 << 20) + 1024)) == -1    # overlapping buffers
    assert "overlap" in lib.moe_last_error().decode()


def test_publish_rejects_misaligned_weights():
    lib = moe.lib()
    h = moe.ExpertHandle()
    h.fmt = moe.MOE_W_BF16
    h.w_gate, h.w_up, h.w_down = 1 << 20, (1 << 20) + 8, 1 << 21
    assert lib.moe_handle_publish(FAKE, 0, ctypes.byref(h), None) == -1
    assert "aligned" in lib.moe_last_error().decode()


def test_route_dispatch_rejects_bad_arguments():
    lib = moe.lib()
    args = lambda **kw: [kw.get(n, d) for n, d in (
        ("logits", FAKE), ("B", 16), ("N", 128), ("k", 8), ("mode", 1), ("k0", 3), ("p", 1.0), ("max_p", 128),
        ("renorm", 1), ("n_valid", None), ("idx", FAKE), ("w", FAKE), ("n_base", None), ("mask", None),
        ("cnt", FAKE), ("offsets", FAKE), ("perm", FAKE), ("active", FAKE), ("T", FAKE), ("stream", None))]
    assert lib.moe_route_dispatch(*args(mode=3)) == -1
    assert lib.moe_route_dispatch(*args(max_p=2)) == -1          # max_p < k0
    assert lib.moe_route_dispatch(*args(max_p=129)) == -1        # max_p > N
    assert lib.moe_route_dispatch(*args(k0=9)) == -1
    assert lib.moe_route_dispatch(*args(p=0.0)) == -1
    assert lib.moe_route_dispatch(*args(perm=None)) == -1
    assert lib.moe_route_dispatch(*args(B=129)) == -2
    assert lib.moe_route_dispatch(*args(N=0)) == -1
