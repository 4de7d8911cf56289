"""Negative controls on the GPU side: the planted mistakes of the oracle
mutants (tests/test_oracle_mutants.py: score faults, dropped or unscaled
gradients, misaligned rows, wrong intra-expert order, off-by-one offsets,
other dot orders, truncating bf16 rounding; tests/test_oracle_staged.py:
shifted send rows, the wrong partition in the expansion, a partition reduce
that ignores partitions, descending partition order in the merge;
tests/test_oracle_padding.py: segments rounded down, padding placed first,
stale padding rows) must each
make the GPU-vs-oracle comparison fail, while the real oracle matches the GPU
bit for bit.  The mistakes live in the oracle, on the CPU; the GPU runs the
real kernels once.  The comparison's bar is zero ulp, so it is below the
smallest fault."""
import numpy as np
import pytest
import torch

import workloads as W
import combine_moe_layout_04_amd as M
from oracle import moe_oracle as O

import test_oracle_mutants as MU
import test_oracle_padding as MP
import test_oracle_staged as MS
from devutil import n_diff, to_dev, to_host

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def weighted():
    """One weighted layer (scores applied in the combine) on the GPU."""
    cfg = W.get_config("qwen3_30b_a3b", T=512)
    inp = W.layer_inputs(cfg, seed=41)
    say(f"negative controls, weighted: T={cfg.T} H={cfg.H} {cfg.dtype}")
    dt = cfg.dtype
    idx = torch.from_numpy(inp.topk_idx).to(DEV)
    w = torch.from_numpy(inp.topk_weights).to(DEV)
    x, y, g = (to_dev(a, dt, DEV) for a in (inp.x, inp.y, inp.g))
    h = M.moe_layout(idx, cfg.E, cfg.P)
    recv, sc = M.moe_dispatch(h, x, w, recv_scores=True)
    out = M.moe_combine(h, y, w)
    gy, gw = M.moe_combine_bwd(h, g, w, y, grad_w=True)
    assert h.check() == 0
    fields = {f: h.field(f).cpu().numpy() for f in ("recv_pos", "expert_offset", "token_slot")}
    res = dict(recv=to_host(recv, dt), sc=sc.cpu().numpy(), out=to_host(out, dt), gy=to_host(gy, dt),
               gw=gw.cpu().numpy(), **fields)
    return cfg, inp, O.layout(inp.topk_idx, cfg.E, cfg.P), res


@pytest.fixture(scope="module")
def absorbed():
    """One layer with scores absorbed before W2 (scaled dispatch, plain combine)."""
    cfg = W.get_config("diffusion_gemma", T=512)
    inp = W.layer_inputs(cfg, seed=42)
    say(f"negative controls, absorbed: T={cfg.T} H={cfg.H} {cfg.dtype}")
    dt = cfg.dtype
    idx = torch.from_numpy(inp.topk_idx).to(DEV)
    w = torch.from_numpy(inp.topk_weights).to(DEV)
    x, gr = to_dev(inp.x, dt, DEV), to_dev(inp.grad_recv, dt, DEV)
    h = M.moe_layout(idx, cfg.E, cfg.P)
    gx, gs = M.moe_dispatch_bwd(h, gr, w, x, grad_s=True)
    assert h.check() == 0
    return cfg, inp, O.layout(inp.topk_idx, cfg.E, cfg.P), dict(gx=to_host(gx, dt), gs=gs.cpu().numpy())


def differs(got, real, mutant, what):
    assert n_diff(got, real) == 0, f"{what}: the GPU does not match the real oracle"
    assert n_diff(got, mutant) > 0, f"{what}: the comparison cannot tell the mutant from the GPU result"


@pytest.mark.parametrize("mutant", [MU.combine_double_score, MU.combine_rolled_score])
def test_score_faults(weighted, mutant):
    cfg, inp, lay, res = weighted
    w = inp.topk_weights
    differs(res["out"], O.combine(lay, inp.y, cfg.dtype, w), mutant(lay, inp.y, cfg.dtype, w), mutant.__name__)


def test_truncating_bf16_rounding(weighted):
    cfg, inp, lay, res = weighted
    acc = O.combine(lay, O.to_f32(inp.y, "bf16"), "f32", inp.topk_weights)   # the float32 sums
    differs(res["out"], O.combine(lay, inp.y, "bf16", inp.topk_weights), MU.bf16_truncate(acc), "bf16 truncation")


@pytest.mark.parametrize("mutant", [MU.combine_bwd_no_grad_w, MU.combine_bwd_unscaled_rows])
def test_combine_backward_faults(weighted, mutant):
    cfg, inp, lay, res = weighted
    w = inp.topk_weights
    r_gy, r_gw = O.combine_bwd(lay, inp.g, cfg.dtype, w, inp.y)
    m_gy, m_gw = mutant(lay, inp.g, cfg.dtype, w, inp.y)
    assert n_diff(res["gy"], r_gy) == 0 and n_diff(res["gw"], r_gw) == 0
    assert n_diff(res["gy"], m_gy) + n_diff(res["gw"], m_gw) > 0, mutant.__name__


@pytest.mark.parametrize("mutant", [MU.dispatch_misaligned_tokens, MU.dispatch_scores_k_flipped])
def test_dispatch_faults(weighted, mutant):
    cfg, inp, lay, res = weighted
    w = inp.topk_weights
    r_recv, r_sc = O.dispatch(lay, inp.x, cfg.dtype, w)
    m_recv, m_sc = mutant(lay, inp.x, cfg.dtype, w)
    assert n_diff(res["recv"], r_recv) == 0 and n_diff(res["sc"], r_sc) == 0
    assert n_diff(res["recv"], m_recv) + n_diff(res["sc"], m_sc) > 0, mutant.__name__


@pytest.mark.parametrize("mutant", [MU.layout_reversed_within_expert, MU.layout_offset_off_by_one,
                                    MU.layout_missing_last_boundary, MU.layout_slot_global])
def test_layout_faults(weighted, mutant):
    cfg, inp, lay, res = weighted
    bad = mutant(inp.topk_idx, cfg.E, cfg.P)
    names = ("recv_pos", "expert_offset", "token_slot")
    for f in names:
        assert np.array_equal(res[f], np.asarray(getattr(lay, f))), f
    assert any(not np.array_equal(res[f], np.asarray(getattr(bad, f))) for f in names), mutant.__name__


@pytest.mark.parametrize("mutant", [MU.dot_sequential, MU.dot_32_lanes, MU.dot_fold_reversed, MU.dot_lane_carry,
                                    MU.dot_segment_tree, MU.dot_chunk_reversed])
def test_dot_order_faults(weighted, mutant):
    cfg, inp, lay, res = weighted
    a = np.repeat(inp.g, cfg.K, axis=0)
    b = np.asarray(inp.y)[lay.recv_pos.reshape(-1)]
    real = O.canonical_dot(a, b, cfg.dtype).reshape(cfg.T, cfg.K)
    differs(res["gw"], real, mutant(a, b, cfg.dtype).reshape(cfg.T, cfg.K), mutant.__name__)


def test_scaled_backward_forgetting_the_scale(absorbed):
    cfg, inp, lay, res = absorbed
    w = inp.topk_weights
    r_gx, r_gs = O.dispatch_bwd(lay, inp.grad_recv, cfg.dtype, w, inp.x)
    m_gx, _ = MU.dispatch_bwd_forgets_scale(lay, inp.grad_recv, cfg.dtype, w, inp.x)
    assert n_diff(res["gs"], r_gs) == 0
    differs(res["gx"], r_gx, m_gx, "dispatch_bwd without the scale")


@pytest.fixture(scope="module")
def staged():
    """One staged exchange (send, expansion, partition reduce, merge) on the
    GPU, float32 rows so that the merge's summation order shows in its bits."""
    cfg = W.get_config("qwen3_30b_a3b", T=512).with_(dtype="f32")
    inp = W.layer_inputs(cfg, seed=43)
    say(f"negative controls, staged: T={cfg.T} H={cfg.H} {cfg.dtype} P={cfg.P}")
    dt = cfg.dtype
    idx = torch.from_numpy(inp.topk_idx).to(DEV)
    w = torch.from_numpy(inp.topk_weights).to(DEV)
    x, y = to_dev(inp.x, dt, DEV), to_dev(inp.y, dt, DEV)
    h = M.moe_layout(idx, cfg.E, cfg.P)
    n = int(h.field("send_offset")[-1].item())
    S = M.moe_send(h, x)
    recv, _ = M.moe_expand(h, S, w)
    Q = M.moe_reduce_partitions(h, y, w)
    out = M.moe_combine_partitions(h, Q)
    assert h.check() == 0
    res = dict(S=to_host(S[:n], dt), recv=to_host(recv, dt), Q=to_host(Q[:n], dt), out=to_host(out, dt))
    return cfg, inp, O.layout(inp.topk_idx, cfg.E, cfg.P), res


def test_staged_send_shifted_rows(staged):
    cfg, inp, lay, res = staged
    differs(res["S"], O.send(lay, inp.x), MS.send_off_by_one(lay, inp.x), "send")


def test_staged_expand_wrong_partition(staged):
    cfg, inp, lay, res = staged
    S = O.send(lay, inp.x)
    w = inp.topk_weights
    differs(res["recv"], O.expand(lay, S, cfg.dtype, w)[0], MS.expand_wrong_partition(lay, S, cfg.dtype, w)[0],
            "expand")


def test_staged_reduce_ignoring_partitions(staged):
    cfg, inp, lay, res = staged
    w = inp.topk_weights
    differs(res["Q"], O.reduce_partitions(lay, inp.y, cfg.dtype, w),
            MS.reduce_ignores_partition(lay, inp.y, cfg.dtype, w), "reduce_partitions")


def test_staged_merge_descending_order(staged):
    cfg, inp, lay, res = staged
    Q = O.reduce_partitions(lay, inp.y, cfg.dtype, inp.topk_weights)
    differs(res["out"], O.combine_partitions(lay, Q, cfg.dtype), MS.combine_partitions_descending(lay, Q, cfg.dtype),
            "combine_partitions")


PAD_M = 16


@pytest.fixture(scope="module")
def padded():
    """A layout padded to multiples of 16 and its dispatch on the GPU; the
    receive buffer starts full of NaN so that padding rows left unwritten
    would show."""
    cfg = W.get_config("qwen3_30b_a3b", T=512)
    inp = W.layer_inputs(cfg, seed=44)
    say(f"negative controls, padded m={PAD_M}: T={cfg.T} H={cfg.H} {cfg.dtype}")
    dt = cfg.dtype
    idx = torch.from_numpy(inp.topk_idx).to(DEV)
    w = torch.from_numpy(inp.topk_weights).to(DEV)
    h = M.moe_layout(idx, cfg.E, cfg.P, handle=M.Handle(pad_multiple=PAD_M))
    recv = torch.full((h.R, cfg.H), float("nan"), dtype=torch.bfloat16, device=DEV)
    recv, sc = M.moe_dispatch(h, to_dev(inp.x, dt, DEV), w, recv=recv, recv_scores=True)
    assert h.check() == 0
    fields = {f: h.field(f).cpu().numpy() for f in ("expert_offset", "recv_pos", "recv_token", "recv_k")}
    lay = O.layout(inp.topk_idx, cfg.E, cfg.P, PAD_M)
    end = int(lay.expert_offset[-1])
    return cfg, inp, lay, dict(recv=to_host(recv, dt)[:end], sc=sc.cpu().numpy()[:end], end=end, **fields)


@pytest.mark.parametrize("mutant", [MP.layout_floor, MP.layout_pad_at_front])
def test_padded_layout_faults(padded, mutant):
    cfg, inp, lay, res = padded
    bad = mutant(inp.topk_idx, cfg.E, cfg.P, PAD_M)
    names = ("expert_offset", "recv_pos", "recv_token", "recv_k")
    for f in names:
        assert np.array_equal(res[f], np.asarray(getattr(lay, f))), f
    assert any(not np.array_equal(res[f], np.asarray(getattr(bad, f))) for f in names), mutant.__name__


def test_padded_dispatch_stale_padding(padded):
    cfg, inp, lay, res = padded
    w = inp.topk_weights
    r_recv, r_sc = O.dispatch(lay, inp.x, cfg.dtype, w)
    m_recv, _ = MP.dispatch_no_zero_fill(lay, inp.x, cfg.dtype, w)
    end = res["end"]
    assert n_diff(res["sc"], r_sc[:end]) == 0
    differs(res["recv"], r_recv[:end], m_recv[:end], "padded dispatch")
