"""GPU parity of the staged exchange (send buffer per destination partition,
receiver-side expansion, two-level combine) against the CPU oracle.

Bar: send buffer, send_token, expansion and scores bit-exact; partials and the
two-level combine within max-abs 1e-6 (float32) or 1 bf16 ulp, and, by the
float32 contract (same order, separate roundings), bit-identical.
"""
import zlib

import numpy as np
import pytest
import torch

import workloads as W
import combine_moe_layout_04_amd as M
from oracle import moe_oracle as O

from devutil import assert_f32_close, assert_rows_close, n_diff, to_dev, to_host

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)


def run_staged(cfg, inp, tuning=None, parts=("fwd", "bwd")):
    dt = cfg.dtype
    idx = torch.from_numpy(inp.topk_idx).to(DEV)
    w = torch.from_numpy(inp.topk_weights).to(DEV)
    h = M.moe_layout(idx, cfg.E, cfg.P, handle=M.Handle(**(tuning or {})))
    n_send = int(h.field("send_offset")[-1].item())
    res = {"n_send": n_send, "send_token": h.field("send_token")[:n_send].cpu().numpy()}
    if "fwd" in parts:
        x, y = to_dev(inp.x, dt, DEV), to_dev(inp.y, dt, DEV)
        S = M.moe_send(h, x)
        recv, sc = M.moe_expand(h, S, w, scale_rows=cfg.absorbed, recv_scores=True)
        Q = M.moe_reduce_partitions(h, y, None if cfg.absorbed else w)
        out = M.moe_combine_partitions(h, Q)
        res.update(S=to_host(S[:n_send], dt), recv=to_host(recv, dt), scores=sc.cpu().numpy(),
                   Q=to_host(Q[:n_send], dt), out=to_host(out, dt))
    if "bwd" in parts:
        g, gr = to_dev(inp.g, dt, DEV), to_dev(inp.grad_recv, dt, DEV)
        G = M.moe_send(h, g)
        gy, _ = M.moe_expand(h, G, None if cfg.absorbed else w, scale_rows=not cfg.absorbed)
        Qb = M.moe_reduce_partitions(h, gr, w if cfg.absorbed else None)
        gx = M.moe_combine_partitions(h, Qb)
        # the router-side gradient alone, without its rows
        if cfg.absorbed:
            _, dot = M.moe_dispatch_bwd(h, gr, w, to_dev(inp.x, dt, DEV), grad_x=False, grad_s=True)
        else:
            _, dot = M.moe_combine_bwd(h, g, w, to_dev(inp.y, dt, DEV), grad_y=False, grad_w=True)
        res.update(G=to_host(G[:n_send], dt), grad_y=to_host(gy, dt), Qb=to_host(Qb[:n_send], dt),
                   grad_x=to_host(gx, dt), dot=dot.cpu().numpy())
    res["status"] = h.check()
    return res


def oracle_staged(cfg, inp, parts=("fwd", "bwd")):
    dt = cfg.dtype
    lay = O.layout(inp.topk_idx, cfg.E, cfg.P)
    w = inp.topk_weights
    ref = {"n_send": lay.n_send, "send_token": lay.send_token}
    if "fwd" in parts:
        ref["S"] = O.send(lay, inp.x)
        ref["recv"], ref["scores"] = O.expand(lay, ref["S"], dt, w, cfg.absorbed)
        ref["Q"] = O.reduce_partitions(lay, inp.y, dt, None if cfg.absorbed else w)
        ref["out"] = O.combine_partitions(lay, ref["Q"], dt)
        # the staged dispatch delivers the same receive rows as the direct one
        assert np.array_equal(ref["recv"], O.dispatch(lay, inp.x, dt, w, cfg.absorbed)[0])
    if "bwd" in parts:
        ref["G"] = O.send(lay, inp.g)
        ref["grad_y"], _ = O.expand(lay, ref["G"], dt, None if cfg.absorbed else w, not cfg.absorbed)
        ref["Qb"] = O.reduce_partitions(lay, inp.grad_recv, dt, w if cfg.absorbed else None)
        ref["grad_x"] = O.combine_partitions(lay, ref["Qb"], dt)
        if cfg.absorbed:
            ref["dot"] = O.dispatch_bwd(lay, inp.grad_recv, dt, w, inp.x)[1]
        else:
            ref["dot"] = O.combine_bwd(lay, inp.g, dt, w, inp.y)[1]
    return ref


def compare(cfg, res, ref):
    dt = cfg.dtype
    assert res["status"] == 0, res["status"]
    assert res["n_send"] == ref["n_send"]
    assert res.keys() == ref.keys() | {"status"}
    for k in ("send_token", "S", "recv", "scores", "G", "grad_y"):
        if k in ref:
            assert np.array_equal(res[k], ref[k]), f"{k}: {n_diff(res[k], ref[k])} differ"
    for k in ("Q", "out", "Qb", "grad_x"):
        if k in ref:
            assert_rows_close(res[k], ref[k], dt, k)
            assert n_diff(res[k], ref[k]) == 0, f"{k}: {n_diff(res[k], ref[k])} not bit-identical"
    if "dot" in ref:
        assert_f32_close(res["dot"], ref["dot"], "dot")
        assert n_diff(res["dot"], ref["dot"]) == 0


@pytest.mark.parametrize("name", ["tiny", "qwen3_30b_a3b", "skewed_literal", "skewed_calibrated",
                                  "deepseek_v3", "diffusion_gemma"])
@pytest.mark.parametrize("part", ["fwd", "bwd"])
def test_staged_full_size(name, part):
    cfg = W.get_config(name)
    say(f"staged {part} {name} T={cfg.T} H={cfg.H} {cfg.dtype} E={cfg.E} P={cfg.P} K={cfg.K}")
    inp = W.layer_inputs(cfg, seed=1)
    compare(cfg, run_staged(cfg, inp, parts=(part,)), oracle_staged(cfg, inp, parts=(part,)))


RAGGED = [("tiny", dict(T=37)), ("tiny", dict(T=129, H=12)), ("qwen3_30b_a3b", dict(T=131, H=1032)),
          ("diffusion_gemma", dict(T=67, H=520)), ("deepseek_v3", dict(T=45, H=4104)),
          ("qwen3_30b_a3b", dict(T=19, H=8712))]


@pytest.mark.parametrize("name,over", RAGGED)
@pytest.mark.parametrize("tuning", [dict(), dict(nontemporal=0, waves_per_block=1),
                                    dict(nontemporal=1, waves_per_block=2),
                                    dict(nontemporal=2, waves_per_block=8)])
def test_staged_ragged(name, over, tuning):
    cfg = W.get_config(name, **over)
    say(f"staged ragged {name} {over} {tuning}")
    inp = W.layer_inputs(cfg, seed=4)
    compare(cfg, run_staged(cfg, inp, tuning), oracle_staged(cfg, inp))


@pytest.mark.parametrize("case", ["dup", "one_partition", "expert_per_partition", "single"])
@pytest.mark.parametrize("absorbed", [False, True])
def test_staged_edge_cases(case, absorbed):
    rng = np.random.default_rng(zlib.crc32(f"staged/{case}/{absorbed}".encode()))
    if case == "dup":
        T, K, E, P = 70, 4, 6, 3
        idx = rng.integers(0, E, size=(T, K)).astype(np.int32)
    elif case == "one_partition":
        T, K, E, P = 90, 3, 12, 1
        idx = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    elif case == "expert_per_partition":
        T, K, E, P = 50, 5, 8, 8
        idx = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    else:
        T, K, E, P = 1, 1, 1, 1
        idx = np.zeros((1, 1), np.int32)
    H = 40
    say(f"staged edge {case} absorbed={absorbed}")
    cfg = W.get_config("tiny").with_(T=T, H=H, dtype="bf16", E=E, P=P, K=K, absorbed=absorbed)
    w = rng.random((T, K)).astype(np.float32)

    def rows(n):
        return O.f32_to_bf16(rng.standard_normal((n, H)).astype(np.float32))

    inp = W.LayerInputs(cfg, idx, w, rows(T), rows(T * K), rows(T), rows(T * K))
    compare(cfg, run_staged(cfg, inp), oracle_staged(cfg, inp))


def test_staged_validation():
    from combine_moe_layout_04_amd._lib import lib
    import ctypes
    L = lib()
    idx = torch.zeros((8, 2), dtype=torch.int32, device=DEV)
    idx[:, 1] = 3
    h = M.moe_layout(idx, 4, 2)
    assert M.moe_send_capacity(h) == 16
    p = ctypes.c_void_p(h.workspace.data_ptr())
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert L.moe_send(h.ptr, p, 1, 64, p, 15, s) == -2           # capacity below T*min(K,P)
    assert L.moe_expand(h.ptr, p, 1, 64, 16, None, 1, p, None, s) == -1   # scaling needs weights
    assert L.moe_reduce_partitions(h.ptr, p, 1, 64, None, p, 8, s) == -2
    assert L.moe_combine_partitions(h.ptr, None, 1, 64, 16, p, s) == -1
    assert L.moe_combine_bwd(h.ptr, p, 1, 64, None, None, None, None, s) == -1  # neither output
    assert L.moe_dispatch_bwd(h.ptr, p, 1, 64, None, None, None, None, s) == -1
    assert h.check() == 0


def test_staged_empty_batch():
    idx = torch.zeros((0, 4), dtype=torch.int32, device=DEV)
    h = M.moe_layout(idx, 16, 4)
    assert M.moe_send_capacity(h) == 0
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV)
    S = M.moe_send(h, x)
    recv, _ = M.moe_expand(h, S)
    Q = M.moe_reduce_partitions(h, recv)
    out = M.moe_combine_partitions(h, Q)
    assert S.shape == (0, 64) and recv.shape == (0, 64) and out.shape == (0, 64)
    assert h.check() == 0
