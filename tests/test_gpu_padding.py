"""GPU parity of padded layouts (expert segments padded to a multiple, zero
rows and zero scores in the padding) and of varying token counts on one
workspace, against the CPU oracle.

Bar: layout fields, receive rows (real and padding), scores bit-exact;
sums and gradients within max-abs 1e-6 (float32) or 1 bf16 ulp and, by the
float32 contract, bit-identical.  Rows past the last padded segment must be
left untouched (checked against a sentinel the test writes first), and
calls that read receive rows must not read padding (it holds NaN here).
"""
import numpy as np
import pytest
import torch

import workloads as W
import combine_moe_layout_04_amd as M
from oracle import moe_oracle as O

from devutil import assert_f32_close, assert_rows_close, n_diff, to_dev, to_host

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

LAYOUT_FIELDS = ["num_tokens_per_expert", "num_tokens_per_rank", "is_token_in_rank",
                 "expert_offset", "rank_offset", "send_offset", "token_slot",
                 "recv_pos", "recv_token", "recv_k"]
SENTINEL_BF16 = np.uint16(0x7FA5)           # a NaN pattern no kernel writes
SENTINEL_F32 = np.uint32(0x7FA5A5A5)


def say(msg):
    print(msg, flush=True)


def sentinel_rows(n, H, dtype):
    if dtype == "bf16":
        return np.full((n, H), SENTINEL_BF16, np.uint16)
    return np.full((n, H), SENTINEL_F32, np.uint32).view(np.float32)


def nan_padded(lay, un, rows_un, dtype):
    """Unpadded receive rows moved to their padded rows; NaN in every other row."""
    nan = np.uint16(0x7FC0) if dtype == "bf16" else np.float32(np.nan)
    out = np.full((lay.R, rows_un.shape[1]), nan, dtype=rows_un.dtype)
    out[lay.recv_pos.ravel()] = rows_un[un.recv_pos.ravel()]
    return out


def same_bits(a, b):
    a, b = np.asarray(a), np.asarray(b)
    if a.dtype == np.float32:
        a, b = a.view(np.uint32), b.view(np.uint32)
    return a.shape == b.shape and np.array_equal(a, b)


def check_receive_rows(got, ref, lay, dtype, what):
    """Rows [0, expert_offset[E]) equal the oracle's (pairs and zero padding);
    the rest still hold the sentinel."""
    end = int(lay.expert_offset[-1])
    assert same_bits(got[:end], ref[:end]), f"{what}: {n_diff(got[:end], ref[:end])} differ"
    tail = sentinel_rows(lay.R - end, got.shape[1], dtype)
    assert same_bits(got[end:], tail), f"{what}: rows past the last segment were written"


def run_and_check(cfg, inp, m, tuning=None):
    dt = cfg.dtype
    lay = O.layout(inp.topk_idx, cfg.E, cfg.P, m)
    un = O.layout(inp.topk_idx, cfg.E, cfg.P)
    idx = torch.from_numpy(inp.topk_idx).to(DEV)
    w = torch.from_numpy(inp.topk_weights).to(DEV)
    x, g = to_dev(inp.x, dt, DEV), to_dev(inp.g, dt, DEV)
    h = M.moe_layout(idx, cfg.E, cfg.P, handle=M.Handle(pad_multiple=m, **(tuning or {})))
    assert h.R == lay.R == M.moe_recv_capacity(h)
    for f in LAYOUT_FIELDS:
        got = h.field(f).cpu().numpy()
        assert np.array_equal(got, np.asarray(getattr(lay, f)).astype(got.dtype)), f

    H = cfg.H
    wn = inp.topk_weights
    # dispatch (direct and staged) into buffers that hold a sentinel
    ref_recv, ref_sc = O.dispatch(lay, inp.x, dt, wn, cfg.absorbed)
    for how in ("direct", "staged"):
        recv = to_dev(sentinel_rows(lay.R, H, dt), dt, DEV)
        sc = torch.from_numpy(np.full(lay.R, -7.0, np.float32)).to(DEV)
        if how == "direct":
            M.moe_dispatch(h, x, w, scale_rows=cfg.absorbed, recv=recv, recv_scores=sc)
        else:
            M.moe_expand(h, M.moe_send(h, x), w, scale_rows=cfg.absorbed, recv=recv, recv_scores=sc)
        check_receive_rows(to_host(recv, dt), ref_recv, lay, dt, f"{how} recv")
        end = int(lay.expert_offset[-1])
        s = sc.cpu().numpy()
        assert same_bits(s[:end], ref_sc[:end]) and np.all(s[end:] == -7.0), f"{how} scores"

    # readers: NaN in the padding must not matter
    y = nan_padded(lay, un, inp.y, dt)
    gr = nan_padded(lay, un, inp.grad_recv, dt)
    yd, grd = to_dev(y, dt, DEV), to_dev(gr, dt, DEV)
    wc = None if cfg.absorbed else wn
    out = M.moe_combine(h, yd, None if cfg.absorbed else w)
    assert_rows_close(to_host(out, dt), O.combine(lay, y, dt, wc), dt, "combine")
    assert n_diff(to_host(out, dt), O.combine(lay, y, dt, wc)) == 0
    gx, gs = M.moe_dispatch_bwd(h, grd, w if cfg.absorbed else None, x if cfg.absorbed else None,
                                grad_s=cfg.absorbed)
    rgx, rgs = O.dispatch_bwd(lay, gr, dt, wn if cfg.absorbed else None, inp.x if cfg.absorbed else None)
    assert n_diff(to_host(gx, dt), rgx) == 0, "dispatch_bwd"
    if cfg.absorbed:
        assert_f32_close(gs.cpu().numpy(), rgs, "grad_s")
        assert n_diff(gs.cpu().numpy(), rgs) == 0
    Q = M.moe_reduce_partitions(h, yd, None if cfg.absorbed else w)
    two = M.moe_combine_partitions(h, Q)
    assert n_diff(to_host(two, dt), O.combine_partitions(lay, O.reduce_partitions(lay, y, dt, wc), dt)) == 0

    # combine backward: zero gradient rows in the padding, sentinel past it
    grad_y = to_dev(sentinel_rows(lay.R, H, dt), dt, DEV)
    _, gw = M.moe_combine_bwd(h, g, None if cfg.absorbed else w, None if cfg.absorbed else yd,
                              grad_y=grad_y, grad_w=not cfg.absorbed)
    rgy, rgw = O.combine_bwd(lay, inp.g, dt, wc, None if cfg.absorbed else y)
    check_receive_rows(to_host(grad_y, dt), rgy, lay, dt, "grad_y")
    if not cfg.absorbed:
        assert_f32_close(gw.cpu().numpy(), rgw, "grad_w")
        assert n_diff(gw.cpu().numpy(), rgw) == 0
    assert h.check() == 0


@pytest.mark.parametrize("name", ["tiny", "qwen3_30b_a3b", "deepseek_v3", "diffusion_gemma",
                                  "skewed_literal", "skewed_calibrated"])
@pytest.mark.parametrize("m", [16, 128])
def test_padded_full_size(name, m):
    cfg = W.get_config(name)
    say(f"padded {name} m={m} T={cfg.T} H={cfg.H} E={cfg.E} P={cfg.P} K={cfg.K}")
    run_and_check(cfg, W.layer_inputs(cfg, seed=2), m)


RAGGED = [("tiny", dict(T=37)), ("tiny", dict(T=129, H=12)), ("qwen3_30b_a3b", dict(T=70, H=40)),
          ("diffusion_gemma", dict(T=67, H=520)), ("deepseek_v3", dict(T=45, H=4104))]


@pytest.mark.parametrize("name,over", RAGGED)
@pytest.mark.parametrize("m", [1, 2, 3, 64, 1024])
def test_padded_ragged(name, over, m):
    cfg = W.get_config(name, **over)
    say(f"padded ragged {name} {over} m={m}")
    run_and_check(cfg, W.layer_inputs(cfg, seed=6), m)


@pytest.mark.parametrize("tuning", [dict(layout_pairs=4096, waves_per_block=1),
                                    dict(layout_pairs=2048, chunks_per_lane=2, waves_per_block=8),
                                    dict(chunks_per_lane=4, waves_per_block=2, nontemporal=0)])
def test_padded_layout_tunings(tuning):
    cfg = W.get_config("qwen3_30b_a3b", T=3001)
    say(f"padded tunings {tuning}")
    run_and_check(cfg, W.layer_inputs(cfg, seed=7), 32, tuning)


def test_padded_edge_cases():
    rng = np.random.default_rng(99)
    cases = [  # T, K, E, P, idx
        (1, 1, 1, 1, np.zeros((1, 1), np.int32)),
        (40, 2, 8, 8, np.full((40, 2), 5, np.int32)),                      # one expert holds all
        (64, 1, 64, 8, np.arange(64, dtype=np.int32).reshape(64, 1)),      # one pair per expert
        (30, 4, 6, 3, rng.integers(0, 6, size=(30, 4)).astype(np.int32)),  # duplicates
    ]
    for T, K, E, P, idx in cases:
        for m in (4, 7):
            say(f"padded edge T={T} K={K} E={E} P={P} m={m}")
            cfg = W.get_config("tiny").with_(T=T, H=24, dtype="bf16", E=E, P=P, K=K, absorbed=False)
            w = rng.random((T, K)).astype(np.float32)

            def rows(n):
                return O.f32_to_bf16(rng.standard_normal((n, 24)).astype(np.float32))

            run_and_check(cfg, W.LayerInputs(cfg, idx, w, rows(T), rows(T * K), rows(T), rows(T * K)), m)


def test_varying_token_counts_reuse_one_workspace_and_buffers():
    """One handle, one workspace and one set of receive / token buffers sized
    for the largest batch serve every smaller one; a larger batch is refused
    on the host before anything is launched."""
    base = W.get_config("qwen3_30b_a3b")
    m, T_max = 16, base.T
    K, E, P, H = base.K, base.E, base.P, base.H
    h = M.Handle(pad_multiple=m)
    ws = torch.empty(M.moe_workspace_size(T_max, K, E, P, m), dtype=torch.uint8, device=DEV)
    cap = O.recv_capacity(T_max, K, E, m)
    recv_big = torch.empty((cap, H), dtype=torch.bfloat16, device=DEV)
    sc_big = torch.empty(cap, dtype=torch.float32, device=DEV)
    out_big = torch.empty((T_max, H), dtype=torch.bfloat16, device=DEV)
    for T in (T_max, 1, 777, 0, 2048, T_max - 1):
        cfg = base.with_(T=T)
        say(f"varying T={T}")
        inp = W.layer_inputs(cfg, seed=T)
        lay = O.layout(inp.topk_idx, E, P, m)
        M.moe_layout(torch.from_numpy(inp.topk_idx).to(DEV), E, P, handle=h, workspace=ws)
        assert h.workspace is ws and h.R == lay.R <= cap
        w = torch.from_numpy(inp.topk_weights).to(DEV)
        recv, sc = recv_big[:h.R], sc_big[:h.R]
        M.moe_dispatch(h, to_dev(inp.x, "bf16", DEV), w, recv=recv, recv_scores=sc)
        out = M.moe_combine(h, recv, w, out=out_big[:T])
        ref_recv, ref_sc = O.dispatch(lay, inp.x, "bf16", inp.topk_weights)
        end = int(lay.expert_offset[-1])
        assert same_bits(to_host(recv, "bf16")[:end], ref_recv[:end])
        assert same_bits(sc.cpu().numpy()[:end], ref_sc[:end])
        ref_out = O.combine(lay, ref_recv, "bf16", inp.topk_weights)
        assert n_diff(to_host(out, "bf16"), ref_out) == 0
        assert h.check() == 0
    big = torch.zeros((T_max + 1, K), dtype=torch.int32, device=DEV)
    with pytest.raises(M.MoeError):
        M.moe_layout(big, E, P, handle=h, workspace=ws)


@pytest.mark.parametrize("m", [1, 8])
def test_empty_batch_every_call(m):
    """T = 0: every call succeeds, reading and writing nothing (torch's empty
    tensors pass NULL data pointers)."""
    E, P, K, H = 16, 4, 2, 32
    h = M.moe_layout(torch.zeros((0, K), dtype=torch.int32, device=DEV), E, P,
                     handle=M.Handle(pad_multiple=m))
    assert h.R == E * (m - 1)
    x = torch.zeros((0, H), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((0, K), dtype=torch.float32, device=DEV)
    rows = torch.full((h.R, H), 3.0, dtype=torch.bfloat16, device=DEV)
    recv, sc = M.moe_dispatch(h, x, w, scale_rows=True, recv_scores=True)
    M.moe_combine(h, rows, w)
    gy, gw = M.moe_combine_bwd(h, x, w, rows, grad_w=True)
    gx, gs = M.moe_dispatch_bwd(h, rows, w, x, grad_s=True)
    M.moe_combine_bwd(h, x, w, rows, grad_y=False, grad_w=True)
    M.moe_dispatch_bwd(h, rows, w, x, grad_x=False, grad_s=True)
    M.moe_combine_partitions(h, M.moe_reduce_partitions(h, rows, w))
    M.moe_expand(h, M.moe_send(h, x), w, scale_rows=True, recv_scores=True)
    assert gw.shape == (0, K) and gs.shape == (0, K) and gx.shape == (0, H)
    assert h.check() == 0
    assert torch.all(rows == 3.0)                      # the receive rows were not touched
