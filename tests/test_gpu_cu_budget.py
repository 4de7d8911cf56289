"""The exchange on a CU-budget stream (a hardware CU mask), alone and beside a
GEMM on the other CUs: results stay bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import workloads as W
import combine_moe_layout_04_amd as M
from oracle import moe_oracle as O

from devutil import n_diff, to_dev, to_host

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)


def exchange(cfg, inp):
    """Layout, dispatch, combine and both backward passes on the current stream."""
    idx = torch.from_numpy(inp.topk_idx).to(DEV)
    w = torch.from_numpy(inp.topk_weights).to(DEV)
    dt = cfg.dtype
    x, y, g, gr = (to_dev(a, dt, DEV) for a in (inp.x, inp.y, inp.g, inp.grad_recv))
    h = M.moe_layout(idx, cfg.E, cfg.P)
    recv, sc = M.moe_dispatch(h, x, w, recv_scores=True)
    out = M.moe_combine(h, y, w)
    gy, gw = M.moe_combine_bwd(h, g, w, y, grad_w=True)
    gx, _ = M.moe_dispatch_bwd(h, gr)
    return h, dict(recv=recv, sc=sc, out=out, gy=gy, gw=gw, gx=gx)


def check(cfg, inp, res):
    dt = cfg.dtype
    lay = O.layout(inp.topk_idx, cfg.E, cfg.P)
    w = inp.topk_weights
    r_recv, r_sc = O.dispatch(lay, inp.x, dt, w)
    r_gy, r_gw = O.combine_bwd(lay, inp.g, dt, w, inp.y)
    pairs = [("recv", r_recv), ("sc", r_sc), ("out", O.combine(lay, inp.y, dt, w)),
             ("gy", r_gy), ("gw", r_gw), ("gx", O.dispatch_bwd(lay, inp.grad_recv, dt)[0])]
    for k, ref in pairs:
        got = res[k].cpu().numpy() if k in ("sc", "gw") else to_host(res[k], dt)
        assert n_diff(got, ref) == 0, f"{k}: {n_diff(got, ref)} differ"


def test_exchange_on_a_cu_budget():
    cfg = W.get_config("qwen3_30b_a3b")
    inp = W.layer_inputs(cfg, seed=3)
    ncu = torch.cuda.get_device_properties(DEV).multi_processor_count
    for first, count in ((0, 32), (0, 8), (ncu - 64, 64)):
        say(f"budget CUs [{first}, {first + count})")
        bs = M.CuBudgetStream(first, count)
        try:
            with torch.cuda.stream(bs.stream):
                h, res = exchange(cfg, inp)
                assert h.check() == 0
            bs.stream.synchronize()
        finally:
            bs.close()
        check(cfg, inp, res)


def test_exchange_beside_a_gemm_on_the_other_cus():
    cfg = W.get_config("qwen3_30b_a3b")
    inp = W.layer_inputs(cfg, seed=4)
    ncu = torch.cuda.get_device_properties(DEV).multi_processor_count
    a = torch.randn((cfg.R, cfg.H), device=DEV).to(torch.bfloat16)
    b = torch.randn((cfg.H, 1536), device=DEV).to(torch.bfloat16)
    alone = torch.matmul(a, b)
    torch.cuda.synchronize()
    xs, gs = M.CuBudgetStream(0, 64), M.CuBudgetStream(64, ncu - 64)
    try:
        with torch.cuda.stream(gs.stream):
            beside = [torch.matmul(a, b) for _ in range(4)]
        with torch.cuda.stream(xs.stream):
            h, res = exchange(cfg, inp)
            assert h.check() == 0
        torch.cuda.synchronize()
    finally:
        xs.close()
        gs.close()
    check(cfg, inp, res)
    for c in beside:
        assert torch.allclose(c.float(), alone.float(), rtol=1e-2, atol=1e-1)


def test_budget_range_is_checked_on_the_host():
    ncu = torch.cuda.get_device_properties(DEV).multi_processor_count
    for first, count in ((0, ncu + 1), (ncu - 3, 4), (-1, 4), (0, 0), (0, 1), (5, 7)):
        with pytest.raises(M.MoeError):
            M.CuBudgetStream(first, count)
