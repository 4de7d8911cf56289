"""Seeded random shapes through every call, direct and staged, padded or not,
against the CPU oracle: bit-exact layout, rows, sums and dots.  Each case is
small; together they cross the shape parameters that the fixed cases test
one at a time (token count including 0, top-k, experts per partition,
partitions up to 64, row width across segment boundaries, element type,
pad multiple, weighted or absorbed scores, duplicate ids, int64 ids)."""
import zlib

import numpy as np
import pytest
import torch

import workloads as W
import combine_moe_layout_04_amd as M
from oracle import moe_oracle as O

from devutil import n_diff, to_dev, to_host

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
FIELDS = ["num_tokens_per_expert", "num_tokens_per_rank", "is_token_in_rank", "expert_offset",
          "rank_offset", "send_offset", "token_slot", "recv_pos", "recv_token", "recv_k"]


def draw_case(i):
    rng = np.random.default_rng(zlib.crc32(f"random-case-{i}".encode()))
    P = int(rng.choice([1, 2, 4, 8, 16, 64]))
    E = P * int(rng.choice([1, 2, 3, 4, 8]))
    K = int(rng.integers(1, min(E, 9) + 1))
    T = int(rng.choice([0, 1, 2, 7, 33, 64, 65, 130, 257]))
    dtype = str(rng.choice(["f32", "bf16"]))
    per_chunk = 4 if dtype == "f32" else 8
    # chunks per row: up to 200 the register gather runs by default; from 256
    # the LDS-staged one, at one wave per workgroup (256, 896: whole segments)
    # or the row kernels' four (352: half a segment last; 512: 8 segments)
    H = per_chunk * int(rng.choice([1, 3, 63, 64, 65, 130, 200, 256, 352, 512, 896]))
    pad = int(rng.choice([1, 1, 2, 5, 16]))
    absorbed = bool(rng.random() < 0.3)
    dup = bool(rng.random() < 0.25)
    i64 = bool(rng.random() < 0.3)
    if dup:
        idx = rng.integers(0, E, size=(T, K))
    else:
        idx = np.argsort(rng.random((T, E)), axis=1)[:, :K] if T else np.zeros((0, K))
    idx = idx.astype(np.int64 if i64 else np.int32)
    w = rng.random((T, K)).astype(np.float32)

    def rows(n):
        a = rng.standard_normal((n, H)).astype(np.float32)
        return a if dtype == "f32" else O.f32_to_bf16(a)

    cfg = W.get_config("tiny").with_(T=T, H=H, dtype=dtype, E=E, P=P, K=K, absorbed=absorbed)
    return cfg, pad, W.LayerInputs(cfg, idx, w, rows(T), rows(T * K), rows(T), rows(T * K))


@pytest.mark.parametrize("i", range(64))
def test_random_case(i):
    cfg, pad, inp = draw_case(i)
    dt = cfg.dtype
    print(f"case {i}: T={cfg.T} K={cfg.K} E={cfg.E} P={cfg.P} H={cfg.H} {dt} pad={pad} "
          f"absorbed={cfg.absorbed} ids={inp.topk_idx.dtype}", flush=True)
    lay = O.layout(inp.topk_idx, cfg.E, cfg.P, pad)
    un = O.layout(inp.topk_idx, cfg.E, cfg.P)
    h = M.moe_layout(torch.from_numpy(inp.topk_idx).to(DEV), cfg.E, cfg.P, handle=M.Handle(pad_multiple=pad))
    assert h.R == lay.R
    for f in FIELDS:
        got = h.field(f).cpu().numpy()
        assert np.array_equal(got, np.asarray(getattr(lay, f)).astype(got.dtype)), f
    w = torch.from_numpy(inp.topk_weights).to(DEV)
    wn = inp.topk_weights
    x, g = to_dev(inp.x, dt, DEV), to_dev(inp.g, dt, DEV)
    # receive-row inputs at their padded rows (zeros in the padding)
    y = np.zeros((lay.R, cfg.H), inp.y.dtype)
    gr = np.zeros((lay.R, cfg.H), inp.y.dtype)
    y[lay.recv_pos.ravel()] = inp.y[un.recv_pos.ravel()]
    gr[lay.recv_pos.ravel()] = inp.grad_recv[un.recv_pos.ravel()]
    yd, grd = to_dev(y, dt, DEV), to_dev(gr, dt, DEV)
    end = int(lay.expert_offset[-1]) if cfg.T else 0
    sc_mode = cfg.absorbed
    wc = None if sc_mode else wn

    recv, sc = M.moe_dispatch(h, x, w, scale_rows=sc_mode, recv_scores=True)
    r_recv, r_sc = O.dispatch(lay, inp.x, dt, wn, sc_mode)
    assert n_diff(to_host(recv, dt)[:end], r_recv[:end]) == 0, "dispatch"
    assert n_diff(sc.cpu().numpy()[:end], r_sc[:end]) == 0, "scores"
    S = M.moe_send(h, x)
    e_recv, _ = M.moe_expand(h, S, w, scale_rows=sc_mode)
    assert n_diff(to_host(e_recv, dt)[:end], r_recv[:end]) == 0, "expand"

    out = M.moe_combine(h, yd, None if sc_mode else w)
    assert n_diff(to_host(out, dt), O.combine(lay, y, dt, wc)) == 0, "combine"
    two = M.moe_combine_partitions(h, M.moe_reduce_partitions(h, yd, None if sc_mode else w))
    assert n_diff(to_host(two, dt), O.combine_partitions(lay, O.reduce_partitions(lay, y, dt, wc), dt)) == 0

    gy, gw = M.moe_combine_bwd(h, g, None if sc_mode else w, None if sc_mode else yd, grad_w=not sc_mode)
    r_gy, r_gw = O.combine_bwd(lay, inp.g, dt, wc, None if sc_mode else y)
    assert n_diff(to_host(gy, dt)[:end], r_gy[:end]) == 0, "grad_y"
    if not sc_mode:
        assert n_diff(gw.cpu().numpy(), r_gw) == 0, "grad_w"
    gx, gs = M.moe_dispatch_bwd(h, grd, w if sc_mode else None, x if sc_mode else None, grad_s=sc_mode)
    r_gx, r_gs = O.dispatch_bwd(lay, gr, dt, wn if sc_mode else None, inp.x if sc_mode else None)
    assert n_diff(to_host(gx, dt), r_gx) == 0, "grad_x"
    if sc_mode:
        assert n_diff(gs.cpu().numpy(), r_gs) == 0, "grad_s"
    assert h.check() == 0
