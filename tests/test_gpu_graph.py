"""The whole step captured in a HIP graph and replayed: every replay must
reproduce the eager results bit for bit.  Between replays the outputs are
cleared and other library work runs eagerly, with synchronisations, so a
replay that leans on state left by the previous one would show."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as W
import combine_moe_layout_04_amd as M
from combine_moe_layout_04_amd._lib import lib

from devutil import to_dev

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)


def make_step(cfg, inp, pad_multiple=1, staged=False, noalloc=False):
    """Device inputs, preallocated outputs, and a closure running one step
    into them (no allocation inside, so it can be captured).  noalloc: the
    layout is moe_layout_noalloc (its histogram in the library's static
    per-device scratch), called through the C ABI."""
    dt = cfg.dtype
    h = M.Handle(pad_multiple=pad_multiple)
    idx = torch.from_numpy(inp.topk_idx).to(DEV)
    w = torch.from_numpy(inp.topk_weights).to(DEV)
    x, g = to_dev(inp.x, dt, DEV), to_dev(inp.g, dt, DEV)
    R = cfg.R + cfg.E * (pad_multiple - 1)
    tdt = x.dtype

    def rows(n):
        return torch.zeros((n, cfg.H), dtype=tdt, device=DEV)

    y = torch.cat([to_dev(inp.y, dt, DEV), rows(R - cfg.R)])
    gr = torch.cat([to_dev(inp.grad_recv, dt, DEV), rows(R - cfg.R)])
    ws = torch.empty(M.moe_workspace_size(cfg.T, cfg.K, cfg.E, cfg.P, pad_multiple),
                     dtype=torch.uint8, device=DEV)
    cap = cfg.T * min(cfg.K, cfg.P)
    out = dict(recv=rows(R), scores=torch.zeros(R, dtype=torch.float32, device=DEV), out=rows(cfg.T),
               grad_y=rows(R), grad_w=torch.zeros((cfg.T, cfg.K), dtype=torch.float32, device=DEV),
               grad_x=rows(cfg.T), S=rows(cap), Q=rows(cap))

    def layout():
        if not noalloc:
            M.moe_layout(idx, cfg.E, cfg.P, handle=h, workspace=ws)
            return
        stream = torch.cuda.current_stream(DEV).cuda_stream
        rc = lib().moe_layout_noalloc(h.ptr, ctypes.c_void_p(idx.data_ptr()), 0, cfg.T, cfg.K, cfg.E, cfg.P,
                                      ctypes.c_void_p(ws.data_ptr()), ws.numel(), ctypes.c_void_p(stream))
        assert rc == 0, rc
        h.workspace, h.T, h.K, h.E, h.P, h.R, h.device = ws, cfg.T, cfg.K, cfg.E, cfg.P, R, DEV

    def step():
        layout()
        if staged:
            M.moe_send(h, x, send=out["S"])
            M.moe_expand(h, out["S"], w, recv=out["recv"], recv_scores=out["scores"])
            M.moe_reduce_partitions(h, y, w, partial=out["Q"])
            M.moe_combine_partitions(h, out["Q"], out=out["out"])
        else:
            M.moe_dispatch(h, x, w, recv=out["recv"], recv_scores=out["scores"])
            M.moe_combine(h, y, w, out=out["out"])
        M.moe_combine_bwd(h, g, w, y, grad_y=out["grad_y"], grad_w=out["grad_w"])
        M.moe_dispatch_bwd(h, gr, grad_x=out["grad_x"])

    return h, out, step


def snapshot(out):
    return {k: v.clone() for k, v in out.items()}


def same(a, b):
    return torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                       b.view(torch.uint8) if b.dtype != torch.uint8 else b)


@pytest.mark.parametrize("pad_multiple,staged,noalloc,T", [(1, False, False, 1024), (16, False, False, 1024),
                                                            (1, True, False, 1024), (1, False, True, 1024),
                                                            (16, True, True, 1024), (1, False, False, 64),
                                                            (1, False, True, 64), (16, True, False, 64)])
def test_step_replays_bitwise(pad_multiple, staged, noalloc, T):
    """noalloc: the layout without a workspace histogram, the caller it is
    for; the layer run between replays also uses it, so the static scratch
    holds another layer's histogram when each replay starts.  T = 64 (512
    pairs, one tile) captures the one-launch layout."""
    cfg = W.get_config("qwen3_30b_a3b", T=T)
    say(f"graph pad={pad_multiple} staged={staged} noalloc={noalloc} T={T}")
    inp = W.layer_inputs(cfg, seed=11)
    h, out, step = make_step(cfg, inp, pad_multiple, staged, noalloc)
    # eager reference
    step()
    torch.cuda.synchronize()
    assert h.check() == 0
    ref = snapshot(out)
    # other work between replays: a second layer with its own handle
    other = W.layer_inputs(W.get_config("qwen3_30b_a3b", T=700), seed=12)
    _, _, other_step = make_step(W.get_config("qwen3_30b_a3b", T=700), other, noalloc=noalloc)

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        step()                      # warm the capture stream
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for v in out.values():
            v.zero_()              # a fill kernel, eager
        other_step()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert h.check() == 0
        for k in ref:
            assert same(out[k], ref[k]), f"replay {rep}: {k} differs from the eager step"
