"""GPU tests of the online precision residency manager (page "DynaExq":
2.2 / 3.2 versioned residency and publish-after-copy, 2.3 / 3.3 pools and the
budget tracker, 2.4 / 3.4 the migration-stream pipeline with backpressure,
2.5 / 3.5 EMA hotness and the hysteresis policy).

Every forward call is checked against the oracle with the version table that
the manager's states say is published (HI -> bf16, anything else -> INT4), so
a handle that ever resolved to a partial or wrong version fails parity.  The
policy's decisions are checked against oracle.residency.select fed with the
scores the GPU computed (fp32 decisions taken in fp32 on both sides), and the
scores against the oracle's EMA fold.
"""
import numpy as np
import pytest
import torch

import aware_expert_routing_amd as moe
import oracle
import synth
from gpu_util import DEV, bf16_dev, build_layer, max_err_over_rms
from oracle import residency as res_oracle

pytestmark = pytest.mark.gpu

N, K, H, I, B = 16, 4, 256, 128, 8
TOL = 2e-2   # INT4 experts in the table


def _setup(seed, n_hi, **kw):
    layer, host_lo = build_layer(N, K, H, I, seed, fmt="bf16", int4_experts=range(N), with_router=False)
    lo = list(layer.experts)
    host_hi, hi_host = [], []
    for e in range(N):
        mats = synth.expert_weights_bf16(seed, e, H, I)
        host_hi.append(dict(fmt=oracle.FMT_BF16, gate=mats[0], up=mats[1], down=mats[2]))
        hi_host.append(moe.pinned_hi_version(moe.ExpertTensors.pack(moe.MOE_W_BF16, *[bf16_dev(m) for m in mats])))
    torch.cuda.synchronize()
    res = moe.Residency(layer, lo, hi_host, n_hi, **kw)
    return layer, res, host_lo, host_hi, hi_host


def _x(seed):
    xb = synth.to_bf16_bits(synth.activations(seed, B, H))
    return synth.bf16_bits_to_f32(xb), bf16_dev(xb)


def _logits(step, phase):
    # Zipf-biased routing whose hot experts change with the phase
    bias = synth.zipf_bias(N, 1.1, seed=7 + phase)
    return (synth.logits(500 + step, B, N, 1.0) + 2.0 * bias[None, :]).astype(np.float32)


def _forward_and_check(layer, res, host_lo, host_hi, x, xd, logits):
    states = res.states()
    table = [host_hi[e] if states[e] == moe.MOE_RES_HI else host_lo[e] for e in range(N)]
    buf = layer.forward(xd, "topk", logits=torch.from_numpy(logits).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.route(logits, K, oea=False)
    assert np.array_equal(buf.route["idx"].cpu().numpy(), ref["idx"])
    yref = oracle.expert_ffn(table, H, I, x, ref["idx"], ref["w"])
    err, rms = max_err_over_rms(buf.y, yref)
    assert err <= TOL * rms, (err, rms)
    return buf


def _check_published_bytes(layer, res, hi_host):
    # every HI handle points into the pool at a block start, and the block
    # holds the pinned version byte for byte (gate | up | down)
    tab = layer.table.cpu().numpy().view(np.uint64).reshape(N, 8)
    base, m = res.arena.data_ptr(), H * I * 2
    arena = res.arena.cpu().numpy()
    for e in res.hi_set():
        g, u, d = int(tab[e, 1]), int(tab[e, 2]), int(tab[e, 3])
        off = g - base
        assert off % res.block_bytes == 0 and 0 <= off < res.arena.numel()
        assert u == g + m and d == g + 2 * m
        assert np.array_equal(arena[off:off + res.hi_bytes], hi_host[e].numpy())


def test_window_steps_follow_the_policy_and_keep_every_forward_exact():
    n_hi, alpha, margin = 4, 0.5, 1.0
    layer, res, host_lo, host_hi, hi_host = _setup(31, n_hi, alpha=alpha, margin=margin)
    try:
        x, xd = _x(31)
        S_dev = np.zeros(N)
        counts = []
        promoted = demoted = 0
        for step in range(18):
            logits = _logits(step, 0 if step < 9 else 1)
            buf = _forward_and_check(layer, res, host_lo, host_hi, x, xd, logits)
            counts.append(buf.disp["cnt"].cpu().numpy().copy())
            before = res.states()
            force = step % 3 == 2
            res.step(buf.disp["cnt"], force=force, wait=True)
            if not force:
                assert res.states() == before
                continue
            S_gpu = res.S_host.numpy().copy()
            np.testing.assert_allclose(S_gpu, res_oracle.ema_fold(S_dev, counts, alpha), rtol=1e-6, atol=1e-6)
            S_dev, counts = S_gpu.astype(np.float64), []
            in_hi = np.array([s in (moe.MOE_RES_HI, moe.MOE_RES_PROMOTING) for s in before])
            target, pro, dem = res_oracle.select(S_gpu, in_hi, n_hi, margin)
            promoted += len(pro)
            demoted += len(dem)
            assert res.hi_set() == set(np.flatnonzero(target).tolist())
            assert all(s in (moe.MOE_RES_LO, moe.MOE_RES_HI) for s in res.states())   # WAIT settles all
            assert res.budget_used() == len(res.hi_set()) * res.block_bytes
            assert res.free_blocks() == n_hi - len(res.hi_set())
            _check_published_bytes(layer, res, hi_host)
        st = res.stats()
        assert st["promotions_published"] == st["promotions_started"] == promoted
        assert st["demotions"] == st["evictions"] == demoted
        assert demoted > 0, "the hot set moved, so hysteresis must have swapped something"
        assert st["bytes_h2d"] == promoted * res.hi_bytes and st["deferred"] == 0
        _forward_and_check(layer, res, host_lo, host_hi, x, xd, _logits(99, 1))
    finally:
        res.close()
    # close() switched everything back to the low versions
    _forward_and_check(layer, res, host_lo, host_hi, x, xd, _logits(100, 1))


def test_budget_backpressure_defers_promotions():
    n_hi = 4
    layer, res, host_lo, host_hi, hi_host = _setup(32, n_hi, alpha=0.0, margin=0.0)
    blk = res.block_bytes
    res.close()
    res = moe.Residency(layer, list(layer.experts), hi_host, n_hi, alpha=0.0, margin=0.0, budget_bytes=2 * blk)
    try:
        x, xd = _x(32)
        buf = _forward_and_check(layer, res, host_lo, host_hi, x, xd, _logits(0, 0))
        res.step(buf.disp["cnt"], force=True, wait=True)
        S_gpu = res.S_host.numpy().copy()
        _, pro, _ = res_oracle.select(S_gpu, np.zeros(N, bool), n_hi, 0.0)
        assert len(pro) >= 3
        assert res.hi_set() == set(pro[:2])                 # admitted hottest first, then the budget refused
        assert res.pending() == len(pro) - 2
        assert res.stats()["deferred"] >= 1
        assert res.budget_used() == 2 * blk and res.free_blocks() == n_hi - 2
        res.step(None, wait=True)                            # still no room: stays queued
        assert res.pending() == len(pro) - 2 and res.hi_set() == set(pro[:2])
        _forward_and_check(layer, res, host_lo, host_hi, x, xd, _logits(1, 0))
        _check_published_bytes(layer, res, hi_host)
    finally:
        res.close()


def test_non_blocking_steps_converge_while_the_layer_runs():
    n_hi, margin = 5, 0.5
    layer, res, host_lo, host_hi, hi_host = _setup(33, n_hi, alpha=0.0, margin=margin)
    try:
        x, xd = _x(33)
        buf = _forward_and_check(layer, res, host_lo, host_hi, x, xd, _logits(0, 0))
        res.step(buf.disp["cnt"], force=True)               # no waiting anywhere below
        for it in range(1, 400):
            _forward_and_check(layer, res, host_lo, host_hi, x, xd, _logits(it, 0))
            res.step(None)
            st = res.stats()
            settled = all(s in (moe.MOE_RES_LO, moe.MOE_RES_HI) for s in res.states())
            if st["decisions"] == 1 and settled and res.pending() == 0:
                break
        else:
            pytest.fail("transitions did not settle")
        S_gpu = res.S_host.numpy().copy()
        target, pro, _ = res_oracle.select(S_gpu, np.zeros(N, bool), n_hi, margin)
        assert res.hi_set() == set(pro)
        _check_published_bytes(layer, res, hi_host)
        _forward_and_check(layer, res, host_lo, host_hi, x, xd, _logits(999, 0))
    finally:
        res.close()


def test_update_cadence():
    layer, res, host_lo, host_hi, hi_host = _setup(34, 2, alpha=0.5, interval_s=0.0)
    try:
        x, xd = _x(34)
        for step in range(4):
            buf = layer.forward(xd, "topk", logits=torch.from_numpy(_logits(step, 0)).to(DEV))
            res.step(buf.disp["cnt"], wait=True)
        assert res.stats()["updates"] == 4 and res.stats()["decisions"] == 4
    finally:
        res.close()
    res = moe.Residency(layer, list(layer.experts), hi_host, 2, interval_s=1e9)
    try:
        for step in range(3):
            buf = layer.forward(xd, "topk", logits=torch.from_numpy(_logits(step, 0)).to(DEV))
            res.step(buf.disp["cnt"], wait=True)
        assert res.stats()["updates"] == 0 and res.hi_set() == set()
        res.step(None, force=True, wait=True)
        assert res.stats()["updates"] == 1 and len(res.hi_set()) == 2
    finally:
        res.close()
