"""CPU-only checks of the C ABI: the library loads, exports every entry point
include/*.h declares, and rejects invalid arguments on the host before
anything is launched (no call here reaches a kernel)."""
import ctypes
import os
import re

import pytest

import aware_expert_routing_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("moe.h", "moe_residency.h", "moe_probe.h")]

FAKE = ctypes.c_void_p(1 << 20)   # never dereferenced: every call below fails validation


def _declared():
    text = "".join(open(h).read() for h in HEADERS)
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


def test_expert_ffn_noalloc_rejects_calls_beyond_its_static_workspace():
    # validation runs before the static workspace is looked up, so no GPU is needed
    lib = moe.lib()
    args = lambda B, k, H, I: (FAKE, 128, H, I, FAKE, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, B, k, FAKE, None)
    assert moe.ffn_workspace_bytes(128, 16, 4096, 1536) > moe.NOALLOC_WORKSPACE_BYTES
    assert lib.moe_expert_ffn_noalloc(*args(128, 16, 4096, 1536)) == -2
    assert "32 MiB" in lib.moe_last_error().decode()
    assert lib.moe_expert_ffn_noalloc(*args(16, 8, 2046, 768)) == -1          # H % 32
    assert lib.moe_expert_ffn_noalloc(*args(200, 8, 2048, 768)) == -2         # B > 128
    no_y = list(args(16, 8, 2048, 768))
    no_y[14] = None
    assert lib.moe_expert_ffn_noalloc(*no_y) == -1
    # the header's limit and the binding's copy agree; the largest benchmarked calls fit
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    assert re.search(r"MOE_FFN_NOALLOC_WORKSPACE_BYTES \(\(size_t\)32 << 20\)", text)
    assert moe.NOALLOC_WORKSPACE_BYTES == 32 << 20
    assert moe.ffn_workspace_bytes(128, 8, 2048, 768) <= moe.NOALLOC_WORKSPACE_BYTES
    assert moe.ffn_workspace_bytes(64, 8, 4096, 1536) <= moe.NOALLOC_WORKSPACE_BYTES


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
        ("renorm", 1), ("n_valid", None), ("k0_by_batch", None), ("idx", FAKE), ("w", FAKE), ("n_base", None), ("mask", None),
        ("cnt", FAKE), ("offsets", FAKE), ("perm", FAKE), ("active", FAKE), ("T", FAKE), ("sync", None),
        ("stream", None))]
    assert lib.moe_route_dispatch(*args(mode=3)) == -1
    assert lib.moe_route_dispatch(*args(max_p=2)) == -1          # max_p < k0
    assert lib.moe_route_dispatch(*args(max_p=129)) == -1        # max_p > N
    assert lib.moe_route_dispatch(*args(k0=9)) == -1
    assert lib.moe_route_dispatch(*args(p=0.0)) == -1
    assert lib.moe_route_dispatch(*args(perm=None)) == -1
    assert lib.moe_route_dispatch(*args(B=129)) == -2
    assert lib.moe_route_dispatch(*args(N=0)) == -1


def test_router_route_dispatch_rejects_bad_arguments():
    # the layer's routing call checks everything before it launches: a
    # missing completion word, the activation type, H, the mode and its knobs,
    # and sizes past the supported batch
    lib = moe.lib()
    args = lambda **kw: [kw.get(n, d) for n, d in (
        ("x", FAKE), ("x_dtype", moe.MOE_DT_BF16), ("w_r", FAKE), ("B", 64), ("H", 2048), ("N", 128), ("k", 8),
        ("mode", 0), ("k0", 0), ("p", 1.0), ("max_p", 128), ("renorm", 1), ("n_valid", None), ("k0_by_batch", None),
        ("logits", FAKE), ("idx", FAKE), ("w", FAKE), ("n_base", None), ("mask", None), ("cnt", FAKE),
        ("offsets", FAKE), ("perm", FAKE), ("active", FAKE), ("T", FAKE), ("sync", FAKE), ("stream", None))]
    f = lib.moe_router_route_dispatch
    assert f(*args(sync=None)) == -1 and "null" in lib.moe_last_error().decode()
    assert f(*args(logits=None)) == -1
    assert f(*args(x_dtype=7)) == -1
    assert f(*args(H=2044)) == -1 and "multiple of 8" in lib.moe_last_error().decode()
    assert f(*args(H=0)) == -1
    assert f(*args(mode=5)) == -1
    assert f(*args(mode=1, k0=0)) == -1
    assert f(*args(mode=1, k0=9)) == -1
    assert f(*args(mode=1, k0=3, p=0.0)) == -1
    assert f(*args(mode=1, k0=3, max_p=2)) == -1
    assert f(*args(mode=1, k0=3, max_p=129)) == -1
    assert f(*args(B=129)) == -2
    assert f(*args(k=0)) == -1


# ---------------------------------------------------------------------------
# residency host objects (include/moe_residency.h): pure host bookkeeping
# ---------------------------------------------------------------------------
ARENA = 1 << 32            # a fake device address: the pool never dereferences it


def test_pool_hands_out_each_block_once_and_rejects_foreign_or_double_frees():
    lib = moe.lib()
    blk = 4096
    pool = moe.pool_create(ARENA, 5 * blk + 100, blk)
    try:
        assert lib.moe_pool_total_blocks(pool) == 5 and lib.moe_pool_block_bytes(pool) == blk
        got = [moe.pool_alloc(pool) for _ in range(5)]
        assert sorted(got) == [ARENA + i * blk for i in range(5)]
        assert moe.pool_alloc(pool) is None                  # exhausted: MOE_EFULL, not an error
        assert lib.moe_pool_free_blocks(pool) == 0
        moe.pool_free(pool, got[2])
        assert moe.pool_alloc(pool) == got[2]                # constant-time reuse of the freed block
        moe.pool_free(pool, got[0])
        with pytest.raises(moe.MoeError):
            moe.pool_free(pool, got[0])                      # double free
        with pytest.raises(moe.MoeError):
            moe.pool_free(pool, ARENA + 17)                  # not a block start
        with pytest.raises(moe.MoeError):
            moe.pool_free(pool, ARENA + 5 * blk)             # past the last block
        with pytest.raises(moe.MoeError):
            moe.pool_free(pool, ARENA - blk)
    finally:
        lib.moe_pool_destroy(pool)


def test_pool_rejects_bad_geometry():
    with pytest.raises(moe.MoeError):
        moe.pool_create(ARENA, 1 << 20, 1000)                # not a multiple of 256
    with pytest.raises(moe.MoeError):
        moe.pool_create(ARENA + 128, 1 << 20, 4096)          # misaligned arena
    with pytest.raises(moe.MoeError):
        moe.pool_create(ARENA, 100, 256)                     # no whole block


def test_budget_tracker_matches_the_budget_model_and_is_thread_safe():
    import threading
    from oracle.residency import Budget

    lib = moe.lib()
    b = moe.budget_create(1000, 300)
    try:
        ref = Budget(1000, 300)
        assert lib.moe_budget_capacity(b) == ref.capacity == 700
        for nbytes in [100, 250, 400, 350, 1, 0, 50]:
            assert moe.budget_try_reserve(b, nbytes) == ref.try_reserve(nbytes)
            assert lib.moe_budget_used(b) == ref.used
        moe.budget_release(b, 250)
        ref.release(250)
        assert lib.moe_budget_used(b) == ref.used
        with pytest.raises(moe.MoeError):
            moe.budget_release(b, ref.used + 1)
        moe.budget_release(b, ref.used)
        # many threads racing for 7-byte reservations never overshoot
        wins = []

        def worker():
            n = 0
            for _ in range(2000):
                n += moe.budget_try_reserve(b, 7)
            wins.append(n)

        ts = [threading.Thread(target=worker) for _ in range(8)]
        [t.start() for t in ts]
        [t.join() for t in ts]
        assert sum(wins) == 700 // 7 and lib.moe_budget_used(b) == 700
    finally:
        lib.moe_budget_destroy(b)
    with pytest.raises(moe.MoeError):
        moe.budget_create(10, 11)


def test_residency_select_matches_the_oracle():
    import numpy as np
    import synth
    from oracle import residency as ref

    r = synth.rng(81)
    for trial in range(400):
        N = int(r.integers(1, 129))
        n_hi = int(r.integers(0, N + 1))
        kind = trial % 4
        if kind == 0:
            S = r.random(N).astype(np.float32)
        elif kind == 1:
            S = (r.integers(0, 6, N) / 4.0).astype(np.float32)          # ties and zeros
        elif kind == 2:
            S = (r.zipf(1.5, N) % 50).astype(np.float32) * np.float32(0.1)
        else:
            S = np.float32(0.3) + (r.integers(-2, 3, N) * np.float32(2.0 ** -24))   # margin rounding cases
        cur = r.random(N) < r.random()
        locked = (r.random(N) < 0.15) if trial % 3 == 0 else None
        margin = float(r.choice([0.0, 0.05, 0.1, 2.0 ** -24, 0.3]))
        got = moe.residency_select(S, cur, n_hi, margin, locked)
        want = ref.select(S, cur, n_hi, margin, locked)
        assert np.array_equal(got[0], want[0]) and got[1] == want[1] and got[2] == want[2], trial


def test_residency_create_rejects_bad_configs():
    lib = moe.lib()
    cfg = moe.ResidencyConfig()
    assert lib.moe_residency_create(None, None) == -1
    out = ctypes.c_void_p()
    cfg.N, cfg.H, cfg.I = 16, 256, 128
    assert lib.moe_residency_create(ctypes.byref(cfg), ctypes.byref(out)) == -1   # null pointers
    assert "null" in moe.lib().moe_last_error().decode()
    cfg.N = 0
    assert lib.moe_residency_create(ctypes.byref(cfg), ctypes.byref(out)) == -1
    cfg.N, cfg.H = 16, 200
    assert lib.moe_residency_create(ctypes.byref(cfg), ctypes.byref(out)) == -1
    assert "multiples of 128" in moe.lib().moe_last_error().decode()
    assert lib.moe_residency_step(None, None, 0) == -1
    assert lib.moe_residency_state(None, 0) == -1


def test_k0_schedule_table():
    t = moe.k0_schedule(8, 16, [(6, 3), (2, 5)], device="cpu").tolist()
    assert len(t) == 17 and t[1] == 8 and t[2:6] == [5] * 4 and t[6:] == [3] * 11
    assert moe.k0_schedule(8, 4, [(1, 2)], device="cpu").tolist() == [8, 8, 2, 2, 2]   # B = 1 stays top-k
    with pytest.raises(ValueError):
        moe.k0_schedule(8, 4, [(2, 9)], device="cpu")


def test_binding_arity_matches_the_headers():
    # every ctypes signature passes exactly the parameters the header declares
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    from aware_expert_routing_amd import _lib
    for name, args, _ in _lib._SIGNATURES:
        m = re.search(r"\b" + name + r"\s*\(([^)]*)\)", text)
        params = [a for a in m.group(1).split(",") if a.strip() and a.strip() != "void"]
        assert len(params) == len(args), name


def test_binding_refuses_short_or_mistyped_device_tables():
    # k0_by_batch is read on the device at index B (the real batch size) and
    # n_valid at index 0: the binding refuses tables that would be read out
    # of bounds, or whose type or placement is wrong, before any library call
    import torch
    logits = torch.zeros(4, 16)
    x = torch.zeros(4, 32)
    w_r = torch.zeros(16, 32)
    bad = [dict(k0_by_batch=torch.zeros(4, dtype=torch.int32)),            # needs B + 1 = 5 entries
           dict(k0_by_batch=torch.zeros(5, dtype=torch.int64)),
           dict(k0_by_batch=torch.zeros(10, dtype=torch.int32)[::2]),      # not contiguous
           dict(n_valid=torch.zeros(0, dtype=torch.int32)),
           dict(n_valid=torch.zeros(1, dtype=torch.float32)),
           dict(n_valid=[4])]
    for kw in bad:
        with pytest.raises(ValueError):
            moe.route_dispatch(logits, 4, "oea", 2, **kw)
        with pytest.raises(ValueError):
            moe.router_route_dispatch(x, w_r, 4, "oea", 2, **kw)
    with pytest.raises(ValueError):
        moe.router_route_dispatch(x, w_r, 4, "oea", 2, sync=torch.zeros(1, dtype=torch.int64))


def test_expert_ffn_phase_events_validates_like_the_ffn_call():
    # the phase-timed copy runs the same validation before anything is recorded or launched
    lib = moe.lib()
    need = moe.ffn_workspace_bytes(16, 8, 2048, 768)
    evs = (ctypes.c_void_p * 4)()
    ev_ptr = ctypes.cast(evs, ctypes.c_void_p)
    args = lambda H, I, ws, events: (FAKE, 128, H, I, FAKE, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, 8, FAKE,
                                     FAKE, ws, events, None)
    assert lib.moe_expert_ffn_phase_events(*args(2048, 768, need, None)) == -1        # no events array
    assert lib.moe_expert_ffn_phase_events(*args(2046, 768, need, ev_ptr)) == -1      # H % 32
    assert lib.moe_expert_ffn_phase_events(*args(2048, 768, need - 1, ev_ptr)) == -1  # workspace
    assert lib.moe_expert_ffn_phase_events(*args(32768, 768, 1 << 40, ev_ptr)) == -2  # beyond limits
