"""Negative controls: oracle copies with one planted mistake each must fail the pins.

These are the fault classes the pages name for their own parity tests
(torchtitan issue, "Tests and verifications": a double-applied and a
misaligned (rolled) router score must be O(1) errors) plus the layout and
backward faults a dispatcher most plausibly gets wrong.  A check that passes
a mutant would be too weak to pin the oracle (the DeepSpeed review thread on
"Avoid collective token preparation for AutoEP DeepEP" catches a tolerance
larger than the update it was meant to see).
"""
import dataclasses

import numpy as np
import pytest

from oracle import moe_oracle as O

import pins

T, K, E, P, H = 12, 3, 8, 2, 16


def routing(seed=0):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.choice(E, size=K, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, K)).astype(np.float32)
    return idx, w


def rows(n, dtype, seed):
    a = np.random.default_rng(seed).standard_normal((n, H)).astype(np.float32)
    return O.f32_to_bf16(a) if dtype == "bf16" else a


# ------------------------------------------------------------ mutants ------

def combine_double_score(lay, y, dtype, w=None):
    return O.combine(lay, y, dtype, None if w is None else w * w)


def combine_rolled_score(lay, y, dtype, w=None):
    return O.combine(lay, y, dtype, None if w is None else np.roll(w, 1, axis=1))


def combine_bwd_no_grad_w(lay, g, dtype, w=None, y=None):
    gy, gw = O.combine_bwd(lay, g, dtype, w, y)
    return gy, (None if gw is None else np.zeros_like(gw))


def combine_bwd_unscaled_rows(lay, g, dtype, w=None, y=None):
    gy, gw = O.combine_bwd(lay, g, dtype, None, None)
    _, gw = O.combine_bwd(lay, g, dtype, w, y)
    return gy, gw


def dispatch_bwd_forgets_scale(lay, gr, dtype, w=None, x=None):
    gx, gs = O.dispatch_bwd(lay, gr, dtype, w, x)
    gx_plain, _ = O.dispatch_bwd(lay, gr, dtype, None, None)
    return (gx_plain if w is not None else gx), gs


def dispatch_misaligned_tokens(lay, x, dtype, w=None, scale_rows=False):
    # bookkeeping off by one token: pair (t,k) lands in the row of (t+1,k)
    shifted = dataclasses.replace(lay, recv_pos=np.roll(lay.recv_pos, 1, axis=0))
    return O.dispatch(shifted, x, dtype, w, scale_rows)


def dispatch_scores_k_flipped(lay, x, dtype, w=None, scale_rows=False):
    # rows right, but the per-row scores take the wrong k
    recv, _ = O.dispatch(lay, x, dtype, w, scale_rows)
    _, sc = O.dispatch(lay, x, dtype, None if w is None else w[:, ::-1].copy(), scale_rows)
    return recv, sc


def layout_reversed_within_expert(idx, E_, P_):
    lay = O.layout(idx, E_, P_)
    pos = lay.recv_pos.copy()
    for e in range(E_):
        lo, hi = lay.expert_offset[e], lay.expert_offset[e + 1]
        m = (pos >= lo) & (pos < hi)
        pos[m] = lo + hi - 1 - pos[m]
    rt = np.empty_like(lay.recv_token)
    rk = np.empty_like(lay.recv_k)
    rt[pos.ravel()] = np.repeat(np.arange(lay.T), lay.K)
    rk[pos.ravel()] = np.tile(np.arange(lay.K), lay.T)
    return dataclasses.replace(lay, recv_pos=pos, recv_token=rt, recv_k=rk)


def layout_offset_off_by_one(idx, E_, P_):
    lay = O.layout(idx, E_, P_)
    eo = lay.expert_offset.copy()
    eo[1:-1] += 1
    return dataclasses.replace(lay, expert_offset=eo)


def layout_missing_last_boundary(idx, E_, P_):
    lay = O.layout(idx, E_, P_)
    eo = lay.expert_offset.copy()
    eo[-1] = eo[-2]
    return dataclasses.replace(lay, expert_offset=eo)


def layout_slot_global(idx, E_, P_):
    lay = O.layout(idx, E_, P_)
    ts = np.where(lay.token_slot >= 0, lay.token_slot + lay.send_offset[:-1][None, :], -1)
    return dataclasses.replace(lay, token_slot=ts.astype(np.int32))


def dot_sequential(a, b, dtype):
    prod = O.to_f32(a, dtype) * O.to_f32(b, dtype)
    acc = np.zeros(prod.shape[0], np.float32)
    for j in range(prod.shape[1]):
        acc = acc + prod[:, j]
    return acc


def _chunk_partials(a, b, dtype, width, reverse_elems=False):
    """Chunk partials padded to segments of ``width`` chunks: [n, NS, width]."""
    V = O.CHUNK_BYTES // (4 if dtype == "f32" else 2)
    n, Hh = np.asarray(a).shape
    NV = Hh // V
    NS = -(-NV // width)
    prod = (O.to_f32(a, dtype) * O.to_f32(b, dtype)).reshape(n, NV, V)
    c = np.zeros((n, NS * width), np.float32)
    order = range(V - 1, -1, -1) if reverse_elems else range(V)
    for i in order:
        c[:, :NV] = c[:, :NV] + prod[:, :, i]
    return c.reshape(n, NS, width)


def _fold(c, steps):
    lane = np.arange(c.shape[-1])
    for s in steps:
        c = c + c[..., lane ^ s]
    return c[..., 0]


def _seq(seg):
    out = np.zeros(seg.shape[0], np.float32)
    for k in range(seg.shape[1]):
        out = out + seg[:, k]
    return out


def dot_32_lanes(a, b, dtype):
    # the canonical algorithm with segments of 32 chunks
    return _seq(_fold(_chunk_partials(a, b, dtype, 32), (16, 8, 4, 2, 1)))


def dot_fold_reversed(a, b, dtype):
    return _seq(_fold(_chunk_partials(a, b, dtype, 64), (1, 2, 4, 8, 16, 32)))


def dot_lane_carry(a, b, dtype):
    # one partial per lane carried across segments, folded once at the end
    V = O.CHUNK_BYTES // (4 if dtype == "f32" else 2)
    n, Hh = np.asarray(a).shape
    NV = Hh // V
    prod = (O.to_f32(a, dtype) * O.to_f32(b, dtype)).reshape(n, NV, V)
    L = np.zeros((n, 64), np.float32)
    for j0 in range(0, NV, 64):
        width = min(64, NV - j0)
        for i in range(V):
            L[:, :width] = L[:, :width] + prod[:, j0:j0 + width, i]
    return _fold(L, (32, 16, 8, 4, 2, 1))


def dot_segment_tree(a, b, dtype):
    # segment values combined pairwise instead of in sequence
    seg = _fold(_chunk_partials(a, b, dtype, 64), (32, 16, 8, 4, 2, 1))
    while seg.shape[1] > 1:
        if seg.shape[1] % 2:
            seg = np.concatenate([seg, np.zeros((seg.shape[0], 1), np.float32)], axis=1)
        seg = seg[:, 0::2] + seg[:, 1::2]
    return seg[:, 0]


def dot_chunk_reversed(a, b, dtype):
    return _seq(_fold(_chunk_partials(a, b, dtype, 64, reverse_elems=True), (32, 16, 8, 4, 2, 1)))


def bf16_truncate(x):
    return (np.ascontiguousarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


# ------------------------------------------------------------- tests -------

@pytest.mark.parametrize("mutant", [combine_double_score, combine_rolled_score])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_score_faults_fail_dense_combine(mutant, dtype):
    idx, w = routing()
    y = rows(T * K, dtype, 1)
    pins.check_combine_dense(O.layout, O.combine, idx, E, P, y, dtype, w)  # real one passes
    with pytest.raises(AssertionError):
        pins.check_combine_dense(O.layout, mutant, idx, E, P, y, dtype, w)


@pytest.mark.parametrize("which", ["combine_bwd_no_grad_w", "combine_bwd_unscaled_rows",
                                   "dispatch_bwd_forgets_scale"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_faults_fail_adjoints(which, dtype):
    idx, _ = routing(2)
    fns = dict(layout_fn=O.layout, dispatch_fn=O.dispatch, combine_fn=O.combine,
               combine_bwd_fn=O.combine_bwd, dispatch_bwd_fn=O.dispatch_bwd)
    pins.check_adjoints(*fns.values(), idx, E, P, H, dtype)
    if which.startswith("combine_bwd"):
        fns["combine_bwd_fn"] = globals()[which]
    else:
        fns["dispatch_bwd_fn"] = globals()[which]
    with pytest.raises(AssertionError):
        pins.check_adjoints(*fns.values(), idx, E, P, H, dtype)


@pytest.mark.parametrize("mutant", [dispatch_misaligned_tokens, dispatch_scores_k_flipped])
def test_dispatch_faults_fail_dense(mutant):
    idx, w = routing(3)
    x = rows(T, "bf16", 4)
    pins.check_dispatch_dense(O.layout, O.dispatch, idx, E, P, x, "bf16", w)
    with pytest.raises(AssertionError):
        pins.check_dispatch_dense(O.layout, mutant, idx, E, P, x, "bf16", w)


@pytest.mark.parametrize("mutant", [layout_reversed_within_expert, layout_offset_off_by_one,
                                    layout_missing_last_boundary, layout_slot_global])
def test_layout_faults_fail_brute_force_and_invariants(mutant):
    idx, _ = routing(4)
    with pytest.raises(AssertionError):
        pins.check_layout_brute(mutant, idx, E, P)
    with pytest.raises(AssertionError):
        pins.check_layout_invariants(mutant(idx, E, P), idx)


@pytest.mark.parametrize("mutant", [dot_sequential, dot_32_lanes, dot_fold_reversed, dot_lane_carry,
                                    dot_segment_tree, dot_chunk_reversed])
def test_dot_order_faults_fail_hand_derived_cases(mutant):
    for dtype in ("f32", "bf16"):
        with pytest.raises(AssertionError):
            pins.check_dot_order(mutant, dtype)


def test_truncating_bf16_fails_torch_pin():
    import torch
    a = np.random.default_rng(0).standard_normal(10_000).astype(np.float32)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f32_to_bf16(a), ref)
    assert not np.array_equal(bf16_truncate(a), ref)


def test_tolerance_sees_the_smallest_score_fault():
    # the GPU bar for bf16 outputs is 1 bf16 ulp; a rolled score must exceed it
    import workloads as W
    cfg = W.get_config("qwen3_30b_a3b").with_(T=64)
    inp = W.layer_inputs(cfg, seed=0)
    lay = O.layout(inp.topk_idx, cfg.E, cfg.P)
    good = O.combine(lay, inp.y, "bf16", inp.topk_weights)
    bad = combine_rolled_score(lay, inp.y, "bf16", inp.topk_weights)
    ulp_gap = np.abs(good.astype(np.int32) - bad.astype(np.int32))
    assert np.max(ulp_gap) > 1
    assert np.mean(ulp_gap > 1) > 0.5
