"""Receive buffers past 4 GiB: every row offset is 64-bit.

A whole layer at T = 32768, K = 8, H = 8256 bf16 puts 262144 receive rows of
16512 bytes in each receive buffer, 4.33 GB, so the last expert segments lie
past byte 2^32 (and a row is 16.1 segments: a partial last segment).  The
layout is compared with the oracle in full.  The rows are compared on a
sample of tokens: every token with a row past 4 GiB (up to 512 of them,
always including the owners of the first such row and of the last row), the
first and last token and 64 random ones.  For the sample the oracle runs on
the sub-problem of those tokens alone (their ids and weights, and the rows
they read), whose results per token and per pair are the full problem's.
Inputs are drawn on the device by torch's seeded generator; none comes from
the library.
"""
import numpy as np
import pytest
import torch

import workloads as W
import combine_moe_layout_04_amd as M
from oracle import moe_oracle as O
from devutil import to_host

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
DT = "bf16"
LAYOUT_FIELDS = ["num_tokens_per_expert", "num_tokens_per_rank", "expert_offset", "rank_offset",
                 "send_offset", "recv_pos", "recv_token", "recv_k"]


def say(msg):
    print(msg, flush=True)


def device_rows(n, H, seed):
    """n x H bf16 rows of N(0,1) draws, made on the device in slices (no
    full-size float32 temporary)."""
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    out = torch.empty((n, H), dtype=torch.bfloat16, device=DEV)
    step = 1 << 15
    for i in range(0, n, step):
        m = min(step, n - i)
        out[i:i + m] = torch.randn((m, H), generator=gen, device=DEV).to(torch.bfloat16)
    return out


def host_rows(t, rows):
    """Rows of a device tensor, in the order given, as host bf16 bits."""
    ix = torch.from_numpy(np.asarray(rows, np.int64).reshape(-1)).to(DEV)
    return to_host(t.index_select(0, ix), DT)


@pytest.mark.parametrize("absorbed,pad", [(False, 1), (True, 1), (False, 128)])
def test_rows_past_4_gib(absorbed, pad):
    cfg = W.get_config("qwen3_30b_a3b").with_(T=32768, H=8256, absorbed=absorbed, renormalize=not absorbed)
    T, H, K, E, P = cfg.T, cfg.H, cfg.K, cfg.E, cfg.P
    row_bytes = H * 2
    first_high = -(-(1 << 32) // row_bytes)   # first row whose byte offset is >= 2^32
    idx_np, w_np = W.routing(cfg, seed=61)
    lay = O.layout(idx_np, E, P, pad_multiple=pad)
    R = len(lay.recv_token)                 # receive rows, padding included
    assert R > first_high
    say(f"rows past 4 GiB: T={T} H={H} bf16, {R} receive rows of {row_bytes} B, absorbed={absorbed} pad={pad}")
    idx = torch.from_numpy(idx_np).to(DEV)
    w = torch.from_numpy(w_np).to(DEV)
    x = device_rows(T, H, 1)
    g = device_rows(T, H, 2)
    y = device_rows(R, H, 3)            # expert outputs; also the receive-row gradient below

    h = M.moe_layout(idx, E, P, handle=M.Handle(pad_multiple=pad))
    assert M.moe_recv_capacity(h) == R
    for f in LAYOUT_FIELDS:
        assert np.array_equal(h.field(f).cpu().numpy(), np.asarray(getattr(lay, f))), f
    if absorbed:
        recv, sc = M.moe_dispatch(h, x, w, scale_rows=True, recv_scores=True)
        out = M.moe_combine(h, y)
        gy, gw = M.moe_combine_bwd(h, g)
        gx, gs = M.moe_dispatch_bwd(h, y, w, x, grad_s=True)
    else:
        recv, sc = M.moe_dispatch(h, x, w, recv_scores=True)
        out = M.moe_combine(h, y, w)
        gy, gw = M.moe_combine_bwd(h, g, w, y, grad_w=True)
        gx, gs = M.moe_dispatch_bwd(h, y)
    torch.cuda.synchronize()
    assert h.check() == 0
    if pad > 1:  # the padding rows of the segments past 4 GiB hold zeros (and zero scores)
        eo = lay.expert_offset
        fill = np.concatenate([np.arange(eo[e] + lay.num_tokens_per_expert[e], eo[e + 1]) for e in range(E)
                               if eo[e + 1] > first_high])
        fill = fill[fill >= first_high]
        assert len(fill) > 0
        for t in (recv, gy):
            assert not host_rows(t, fill).any()
        assert not sc.cpu().numpy()[fill].any()

    rng = np.random.default_rng(7)
    high = np.nonzero((lay.recv_pos >= first_high).any(axis=1))[0]
    owner = lay.recv_token[first_high:]
    must = [int(owner[owner >= 0][0]), int(lay.recv_token[lay.recv_pos.max()]), 0, T - 1]
    pick = rng.choice(high, min(512, len(high)), replace=False)
    S = np.unique(np.concatenate([must, pick, rng.choice(T, 64, replace=False)])).astype(np.int64)
    say(f"{len(high)} tokens own rows past 4 GiB; {len(S)} tokens sampled")
    pos = lay.recv_pos[S]                   # [n, K] rows in the full problem
    sub = O.layout(idx_np[S], E, P, pad_multiple=pad)   # the sampled tokens alone
    spos = sub.recv_pos.reshape(-1)         # their rows in the sub-problem, in (token, k) order
    n = len(S)
    x_s, g_s = host_rows(x, S), host_rows(g, S)
    y_s = np.zeros((len(sub.recv_token), H), np.uint16)
    y_s[spos] = host_rows(y, pos)
    w_s = w_np[S]

    r_recv, r_sc = O.dispatch(sub, x_s, DT, w_s, scale_rows=absorbed)
    assert np.array_equal(host_rows(recv, pos), r_recv[spos]), "dispatch rows"
    assert np.array_equal(sc.cpu().numpy()[pos.reshape(-1)], r_sc[spos]), "receive scores"
    r_out = O.combine(sub, y_s, DT, None if absorbed else w_s)
    assert np.array_equal(host_rows(out, S), r_out), "combine"
    r_gy, r_gw = O.combine_bwd(sub, g_s, DT, None if absorbed else w_s, None if absorbed else y_s)
    assert np.array_equal(host_rows(gy, pos), r_gy[spos]), "combine_bwd rows"
    if not absorbed:
        assert np.array_equal(gw.cpu().numpy()[S], r_gw), "grad_w"
    r_gx, r_gs = O.dispatch_bwd(sub, y_s, DT, w_s if absorbed else None, x_s if absorbed else None)
    assert np.array_equal(host_rows(gx, S), r_gx), "dispatch_bwd rows"
    if absorbed:
        assert np.array_equal(gs.cpu().numpy()[S], r_gs), "grad_s"


@pytest.mark.parametrize("absorbed", [False, True])
def test_staged_rows_past_4_gib(absorbed):
    """The staged exchange with 32 KiB rows (H = 16384 bf16) at T = 32768: the
    send buffer's used rows, the partials and the receive rows all run past
    byte 2^32.  Send and partial rows are matched by (token, partition)
    through each problem's own send_offset and token_slot."""
    cfg = W.get_config("qwen3_30b_a3b").with_(T=32768, H=16384, absorbed=absorbed, renormalize=not absorbed)
    T, H, K, E, P = cfg.T, cfg.H, cfg.K, cfg.E, cfg.P
    R, row_bytes = T * K, H * 2
    first_high = -(-(1 << 32) // row_bytes)
    idx_np, w_np = W.routing(cfg, seed=62)
    lay = O.layout(idx_np, E, P)
    n_send = int(lay.send_offset[P])
    assert n_send > first_high and R > first_high
    say(f"staged rows past 4 GiB: T={T} H={H} bf16, {n_send} send rows, {R} receive rows of {row_bytes} B, "
        f"absorbed={absorbed}")
    idx = torch.from_numpy(idx_np).to(DEV)
    w = torch.from_numpy(w_np).to(DEV)
    x = device_rows(T, H, 11)
    y = device_rows(R, H, 13)

    h = M.moe_layout(idx, E, P)
    for f in LAYOUT_FIELDS + ["token_slot"]:
        assert np.array_equal(h.field(f).cpu().numpy(), np.asarray(getattr(lay, f))), f
    send = M.moe_send(h, x)
    recv, sc = M.moe_expand(h, send, w, scale_rows=absorbed, recv_scores=True)
    partial = M.moe_reduce_partitions(h, y, None if absorbed else w)
    out = M.moe_combine_partitions(h, partial)
    torch.cuda.synchronize()
    assert h.check() == 0

    rng = np.random.default_rng(8)
    srow_all = lay.send_offset[:P][None, :] + lay.token_slot      # send row of (t, r) where token_slot >= 0
    high = np.nonzero(((lay.recv_pos >= first_high).any(axis=1))
                      | ((lay.token_slot >= 0) & (srow_all >= first_high)).any(axis=1))[0]
    must = [int(lay.recv_token[R - 1]), 0, T - 1]
    S = np.unique(np.concatenate([must, rng.choice(high, min(512, len(high)), replace=False),
                                  rng.choice(T, 64, replace=False)])).astype(np.int64)
    say(f"{len(high)} tokens own rows past 4 GiB; {len(S)} tokens sampled")
    sub = O.layout(idx_np[S], E, P)
    on = lay.token_slot[S] >= 0                                     # [n, P], the same in both problems
    assert np.array_equal(on, sub.token_slot >= 0)
    full_send = (lay.send_offset[:P][None, :] + lay.token_slot[S])[on]
    sub_send = (sub.send_offset[:P][None, :] + sub.token_slot)[on]
    assert (full_send >= first_high).any()
    pos = lay.recv_pos[S]
    spos = sub.recv_pos.reshape(-1)
    n = len(S)
    x_s = host_rows(x, S)
    y_s = np.zeros((n * K, H), np.uint16)
    y_s[spos] = host_rows(y, pos)
    w_s = w_np[S]

    r_send = O.send(sub, x_s)
    assert np.array_equal(host_rows(send, full_send), r_send[sub_send]), "send rows"
    r_recv, r_sc = O.expand(sub, r_send, DT, w_s, scale_rows=absorbed)
    assert np.array_equal(host_rows(recv, pos), r_recv[spos]), "expanded rows"
    assert np.array_equal(sc.cpu().numpy()[pos.reshape(-1)], r_sc[spos]), "receive scores"
    r_part = O.reduce_partitions(sub, y_s, DT, None if absorbed else w_s)
    assert np.array_equal(host_rows(partial, full_send), r_part[sub_send]), "partials"
    r_out = O.combine_partitions(sub, r_part, DT)
    assert np.array_equal(host_rows(out, S), r_out), "merged rows"


def test_layout_properties_at_half_a_billion_pairs():
    """A layout of 2^29 - 24 pairs (T = 2^26 - 3, K = 8, E = 128, P = 8: 32768
    tiles, so the histogram is column-scanned), checked on the device through
    properties that define it at any size: the counts and offsets; recv_pos a
    bijection onto [0, R) whose inverse is (recv_token, recv_k); experts in
    ascending order and, inside an expert, pairs in (t, k) order; the send
    schedule (is_token_in_rank, num_tokens_per_rank, send_offset, token_slot
    as each token's rank in its partition's list, send_token its inverse).
    Ids are drawn on the device by torch's seeded generator."""
    T, K, E, P = (1 << 26) - 3, 8, 128, 8
    R, epr = T * K, E // P
    say(f"layout properties T={T} K={K} E={E} P={P}: {R} pairs")
    gen = torch.Generator(device=DEV)
    gen.manual_seed(71)
    idx = torch.randint(0, E, (T, K), generator=gen, device=DEV, dtype=torch.int32)
    h = M.moe_layout(idx, E, P)
    torch.cuda.synchronize()
    assert h.check() == 0
    flat = idx.reshape(-1)
    cnt = torch.bincount(flat, minlength=E)
    assert torch.equal(h.field("num_tokens_per_expert").long(), cnt)
    eo = h.field("expert_offset").long()
    assert eo[0].item() == 0 and torch.equal(eo[1:], torch.cumsum(cnt, 0))
    inv = h.field("recv_token").long() * K + h.field("recv_k").long()      # pair at each receive row
    assert int(inv.min()) >= 0 and int(inv.max()) < R
    rows = torch.arange(R, device=DEV)
    assert torch.equal(h.field("recv_pos").reshape(-1).long()[inv], rows)  # bijection, inverse consistent
    del rows
    e_at = flat[inv]                                                       # expert of each receive row
    assert bool((e_at[1:] >= e_at[:-1]).all())                             # experts ascending
    same = e_at[1:] == e_at[:-1]
    assert bool((inv[1:] > inv[:-1])[same].all())                          # (t, k) order inside an expert
    del e_at, same, inv
    part = (idx // epr).long()
    is_in = torch.zeros((T, P), dtype=torch.bool, device=DEV)
    is_in.scatter_(1, part, True)
    del part
    assert torch.equal(h.field("is_token_in_rank").bool(), is_in)
    ntr = is_in.sum(0)
    assert torch.equal(h.field("num_tokens_per_rank").long(), ntr)
    so = h.field("send_offset").long()
    assert so[0].item() == 0 and torch.equal(so[1:], torch.cumsum(ntr, 0))
    slot = torch.where(is_in, torch.cumsum(is_in, 0, dtype=torch.int32) - 1, torch.full_like(is_in, -1, dtype=torch.int32))
    ts = h.field("token_slot")
    assert torch.equal(ts, slot)
    del slot, is_in
    n_send = int(so[-1])
    st = h.field("send_token")[:n_send].long()
    q = torch.arange(n_send, device=DEV)
    r = torch.searchsorted(so[1:], q, right=True)                          # partition of each send row
    assert torch.equal(ts[st, r].long(), q - so[r])
