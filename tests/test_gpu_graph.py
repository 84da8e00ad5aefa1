"""A whole layer captured into a HIP graph: every replay must reproduce the
eager result bit for bit, with the program's own eager work and device
synchronisation between replays, and the device-side padding mask must let
one captured batch size serve smaller real batches (page "Opportunistic
Expert Activation (OEA) - L2", section 7: padding tokens must not inflate T).
"""
import numpy as np
import pytest
import torch

import aware_expert_routing_amd as moe
import synth
from gpu_util import DEV, build_layer, max_err_over_rms

pytestmark = pytest.mark.gpu


def _same_rows(alone_y, graph_y, pairs):
    """A real batch run alone against the same rows of a padded batch: bit for
    bit, except that a call of at most 8 routed pairs takes the column-split
    path, whose partial sums are added in another order (fp32 rounding)."""
    if pairs > 8:
        return torch.equal(alone_y, graph_y)
    err, rms = max_err_over_rms(alone_y, graph_y.double().cpu().numpy())
    return err <= 1e-5 * rms


def _x(seed, B, H):
    return torch.from_numpy(synth.to_bf16_bits(synth.activations(seed, B, H)).view(np.int16)).to(DEV) \
        .view(torch.bfloat16)


@pytest.mark.parametrize("mode,k0", [("oea", 3), ("topk", 0), ("pruned", 3)])
def test_graph_replays_match_eager(mode, k0):
    N, k, H, I, B = 32, 8, 512, 256, 16
    layer, _ = build_layer(N, k, H, I, 11, fmt="bf16")
    x_static = _x(0, B, H).clone()
    nv = torch.tensor([B], dtype=torch.int32, device=DEV)
    graph = layer.capture(x_static, mode, k0, 1.0, n_valid=nv)
    eager_layer, _ = build_layer(N, k, H, I, 11, fmt="bf16")   # same weights, separate buffers
    for rep, (seed, n_real) in enumerate([(1, 16), (2, 16), (3, 9), (4, 1), (5, 16), (6, 12)]):
        x_static.copy_(_x(seed, B, H))
        nv.fill_(n_real)
        graph.replay()
        torch.cuda.synchronize()
        got = {key: t.clone() for key, t in layer.buffers(B).disp.items()}
        y_graph = layer.buffers(B).y.clone()
        ref = eager_layer.forward(x_static, mode, k0, 1.0, n_valid=nv)
        torch.cuda.synchronize()
        assert torch.equal(y_graph, ref.y), rep
        for key in got:
            assert torch.equal(got[key], ref.disp[key]), (rep, key)
        # padding rows produce exact zeros and the active set is that of the real tokens
        if n_real < B:
            assert torch.count_nonzero(y_graph[n_real:]).item() == 0
            alone = eager_layer.forward(x_static[:n_real].clone(), mode, k0, 1.0)
            torch.cuda.synchronize()
            assert int(alone.disp["T"].item()) == int(got["T"].item())
            assert _same_rows(alone.y, y_graph[:n_real], n_real * k)


def test_graph_follows_the_batch_size_k0_table():
    # one captured graph; each replay's real batch size selects k0 on the device
    N, k, H, I, B = 32, 8, 512, 256, 16
    layer, _ = build_layer(N, k, H, I, 12, fmt="bf16")
    eager_layer, _ = build_layer(N, k, H, I, 12, fmt="bf16")
    table = moe.k0_schedule(k, B, [(2, 5), (6, 3)], device=DEV)
    tab = table.cpu().numpy()
    x_static = _x(20, B, H).clone()
    nv = torch.tensor([B], dtype=torch.int32, device=DEV)
    graph = layer.capture(x_static, "oea", 1, 1.0, n_valid=nv, k0_by_batch=table)
    for rep, (seed, n_real) in enumerate([(21, 16), (22, 1), (23, 4), (24, 9), (25, 16)]):
        x_static.copy_(_x(seed, B, H))
        nv.fill_(n_real)
        graph.replay()
        torch.cuda.synchronize()
        y_graph = layer.buffers(B).y.clone()
        T_graph = int(layer.buffers(B).disp["T"].item())
        alone = eager_layer.forward(x_static[:n_real].clone(), "oea", int(tab[n_real]), 1.0)
        torch.cuda.synchronize()
        assert int(alone.disp["T"].item()) == T_graph, rep
        assert _same_rows(alone.y, y_graph[:n_real], n_real * k), rep


def test_one_graph_for_several_layers():
    # a decode step's layers in one graph: every replay, with eager work and
    # synchronisation between replays, reproduces each layer's eager result
    N, k, H, I, B = 32, 8, 512, 256, 4
    seeds = (31, 32, 33)
    layers = [build_layer(N, k, H, I, s, fmt="bf16")[0] for s in seeds]
    refs = [build_layer(N, k, H, I, s, fmt="bf16")[0] for s in seeds]
    xs = [_x(40 + j, B, H).clone() for j in range(len(layers))]
    graph = moe.capture_layers(list(zip(layers, xs)), "oea", 3, 1.0)
    for rep in range(3):
        for j, x in enumerate(xs):
            x.copy_(_x(100 * rep + j, B, H))
        graph.replay()
        torch.cuda.synchronize()
        for j, (lay, ref) in enumerate(zip(layers, refs)):
            y_graph = lay.buffers(B).y.clone()
            T_graph = int(lay.buffers(B).disp["T"].item())
            eager = ref.forward(xs[j], "oea", 3, 1.0)
            torch.cuda.synchronize()
            assert torch.equal(y_graph, eager.y), (rep, j)
            assert T_graph == int(eager.disp["T"].item()), (rep, j)


@pytest.mark.parametrize("B", [16, 1])
def test_forward_on_a_side_stream(B):
    # the layer launches on the caller's stream: the current stream when none
    # is given (inside `with torch.cuda.stream(s)`), a torch stream, or its raw
    # handle; each gives the default stream's result bit for bit
    N, k, H, I = 32, 8, 512, 256
    layer, _ = build_layer(N, k, H, I, 12, fmt="bf16")
    ref_layer, _ = build_layer(N, k, H, I, 12, fmt="bf16")
    x = _x(7, B, H)
    ref = ref_layer.forward(x, "oea", 3, 1.0)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()   # default priority
    side.wait_stream(torch.cuda.current_stream())
    for how in ("context", "stream", "handle"):
        layer.buffers(B).y.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            xs = x.clone()   # produced on the side stream, consumed there without a sync
            if how == "context":
                out = layer.forward(xs, "oea", 3, 1.0)
            elif how == "stream":
                out = layer.forward(xs, "oea", 3, 1.0, stream=side)
            else:
                out = layer.forward(xs, "oea", 3, 1.0, stream=side.cuda_stream)
        side.synchronize()
        assert torch.equal(out.y, ref.y), how
        for key in ("cnt", "offsets", "perm", "active", "T"):
            assert torch.equal(out.disp[key], ref.disp[key]), (how, key)


@pytest.mark.parametrize("mode,k0,B,n_reals", [("topk", 0, 64, (64, 50, 64)), ("oea", 3, 64, (64, 33, 64)),
                                               ("topk", 0, 100, (100, 61, 17))])
def test_graph_replays_above_48_tokens(mode, k0, B, n_reals):
    # above 48 tokens the layer routes by token groups after the router launch
    # and the last routing workgroup dispatches, counting workgroups in a word
    # it leaves at zero: every replay must still match the eager result
    N, k, H, I = 64, 8, 512, 256
    layer, _ = build_layer(N, k, H, I, 13, fmt="bf16")
    eager_layer, _ = build_layer(N, k, H, I, 13, fmt="bf16")
    x_static = _x(20, B, H).clone()
    nv = torch.tensor([B], dtype=torch.int32, device=DEV)
    graph = layer.capture(x_static, mode, k0, 1.0, n_valid=nv)
    for rep, n_real in enumerate(n_reals):
        x_static.copy_(_x(21 + rep, B, H))
        nv.fill_(n_real)
        graph.replay()
        torch.cuda.synchronize()
        assert int(layer.buffers(B).extra["sync"].item()) == 0, rep
        y_graph = layer.buffers(B).y.clone()
        got = {key: t.clone() for key, t in layer.buffers(B).disp.items()}
        ref = eager_layer.forward(x_static, mode, k0, 1.0, n_valid=nv)
        torch.cuda.synchronize()
        assert torch.equal(y_graph, ref.y), rep
        for key in got:
            assert torch.equal(got[key], ref.disp[key]), (rep, key)
        if n_real < B:
            assert torch.count_nonzero(y_graph[n_real:]).item() == 0
