"""Pins for the oracle's padded layout: every expert segment padded to a
multiple of pad_multiple, with zero rows and zero scores in the padding.

References that are not the oracle's own code:
* explicit Python loops that grow each segment by m until the expert's pairs
  fit, and place the pairs by hand;
* the unpadded layout (itself pinned by brute force): a padded dispatch,
  compacted, is the unpadded dispatch bit for bit, and every call that reads
  receive rows gives the unpadded result even when the padding holds NaN;
* a worked example computed by hand, and a routing that reaches the
  capacity bound T*K + E*(m-1).
Planted mistakes (in oracle copies, on the CPU) must fail these pins.
"""
import numpy as np
import pytest

from oracle import moe_oracle as O


def routing(rng, T, K, E, dup):
    if dup:
        return rng.integers(0, E, size=(T, K)).astype(np.int32)
    return np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)


def rows(rng, n, H, dtype):
    a = rng.standard_normal((n, H)).astype(np.float32)
    return a if dtype == "f32" else O.f32_to_bf16(a)


def brute_padded(idx, E, P, m):
    """Offsets, positions and inverse maps by loops: a segment grows by m
    rows at a time until it holds its expert's pairs."""
    idx = [[int(v) for v in row] for row in np.asarray(idx)]
    T = len(idx)
    K = np.asarray(idx).shape[1] if T else 0
    counts = [0] * E
    for row in idx:
        for e in row:
            counts[e] += 1
    eoff = [0]
    for e in range(E):
        seg = 0
        while seg < counts[e]:
            seg += m
        eoff.append(eoff[-1] + seg)
    cap = T * K + E * (m - 1)
    pos = [[-1] * K for _ in range(T)]
    rtok = [-1] * cap
    rk = [-1] * cap
    for e in range(E):
        p = eoff[e]
        for t in range(T):
            for k in range(K):
                if idx[t][k] == e:
                    pos[t][k] = p
                    rtok[p] = t
                    rk[p] = k
                    p += 1
    epr = E // P
    return dict(expert_offset=np.array(eoff, np.int32),
                rank_offset=np.array([eoff[r * epr] for r in range(P + 1)], np.int32),
                recv_pos=np.array(pos, np.int32).reshape(T, K),
                recv_token=np.array(rtok, np.int32), recv_k=np.array(rk, np.int32),
                num_tokens_per_expert=np.array(counts, np.int32), cap=cap)


def check_padded_layout(layout_fn, idx, E, P, m):
    lay = layout_fn(idx, E, P, m)
    ref = brute_padded(idx, E, P, m)
    assert lay.R == ref["cap"]
    for f in ("expert_offset", "rank_offset", "recv_pos", "recv_token", "recv_k", "num_tokens_per_expert"):
        got = np.asarray(getattr(lay, f))
        assert got.shape == ref[f].shape and np.array_equal(got, ref[f]), f
    # the send schedule does not depend on the padding
    un = layout_fn(idx, E, P, 1)
    for f in ("num_tokens_per_rank", "is_token_in_rank", "send_offset", "token_slot", "send_token"):
        assert np.array_equal(getattr(lay, f), getattr(un, f)), f


def check_padded_dispatch(layout_fn, dispatch_fn, idx, E, P, m, x, dtype, w, scale):
    """Compacting the padded receive rows gives the unpadded ones; padding
    rows are zero with zero scores."""
    lay, un = layout_fn(idx, E, P, m), layout_fn(idx, E, P, 1)
    rp, sp = dispatch_fn(lay, x, dtype, w, scale)
    ru, su = dispatch_fn(un, x, dtype, w, scale)
    assert rp.shape[0] == lay.R
    assert np.array_equal(rp[lay.recv_pos.ravel()], ru[un.recv_pos.ravel()])
    pad = pad_rows_by_loop(lay)
    assert np.all(rp[pad] == 0)
    if w is not None:
        assert np.array_equal(sp[lay.recv_pos.ravel()], su[un.recv_pos.ravel()])
        assert np.all(sp[pad] == 0) and not np.any(np.signbit(sp[pad]))


def pad_rows_by_loop(lay):
    out = []
    for e in range(lay.E):
        used = int(lay.num_tokens_per_expert[e])
        out += list(range(int(lay.expert_offset[e]) + used, int(lay.expert_offset[e + 1])))
    return np.array(out, np.int64)


def nan_padded(lay, un, y_un, dtype):
    """The unpadded receive rows moved to their padded positions, NaN elsewhere."""
    nan = np.float32(np.nan) if dtype == "f32" else np.uint16(0x7FC0)
    y = np.full((lay.R, y_un.shape[1]), nan, dtype=y_un.dtype)
    y[lay.recv_pos.ravel()] = y_un[un.recv_pos.ravel()]
    return y


SHAPES = [(1, 1, 1, 1), (9, 2, 4, 2), (33, 3, 12, 4), (40, 4, 8, 8), (60, 8, 32, 8), (17, 5, 20, 1)]
MULTIPLES = [1, 2, 3, 4, 8, 16]


@pytest.mark.parametrize("T,K,E,P", SHAPES)
@pytest.mark.parametrize("m", MULTIPLES)
@pytest.mark.parametrize("dup", [False, True])
def test_padded_layout_brute_force(T, K, E, P, m, dup):
    rng = np.random.default_rng(T * 1000 + m * 7 + dup)
    idx = routing(rng, T, K, E, dup)
    check_padded_layout(O.layout, idx, E, P, m)
    lay = O.layout(idx, E, P, m)
    assert np.all(lay.expert_offset % m == 0)
    assert lay.expert_offset[-1] <= lay.R


def test_pad_multiple_one_is_the_unpadded_layout():
    rng = np.random.default_rng(5)
    idx = routing(rng, 50, 4, 16, False)
    a, b = O.layout(idx, 16, 4), O.layout(idx, 16, 4, 1)
    for f in a.__dataclass_fields__:
        assert np.array_equal(np.asarray(getattr(a, f)), np.asarray(getattr(b, f))), f
    assert a.R == 200


def test_worked_example():
    """E=4 experts on P=2 partitions, m=4, three tokens, top-2:
    t0 -> (0, 1), t1 -> (0, 2), t2 -> (1, 0).  Expert 0 holds (0,0), (1,0),
    (2,1); expert 1 holds (0,1), (2,0); expert 2 holds (1,1); expert 3 none.
    Segments 3->4, 2->4, 1->4, 0->0 rows: offsets 0, 4, 8, 12, 12."""
    idx = np.array([[0, 1], [0, 2], [1, 0]], np.int32)
    lay = O.layout(idx, 4, 2, 4)
    assert lay.expert_offset.tolist() == [0, 4, 8, 12, 12]
    assert lay.rank_offset.tolist() == [0, 8, 12]
    assert lay.recv_pos.tolist() == [[0, 4], [1, 8], [5, 2]]
    assert lay.R == 6 + 4 * 3
    assert lay.recv_token.tolist() == [0, 1, 2, -1, 0, 2, -1, -1, 1] + [-1] * 9
    assert lay.recv_k.tolist() == [0, 0, 1, -1, 1, 0, -1, -1, 1] + [-1] * 9
    assert lay.padding_rows().tolist() == [3, 6, 7, 9, 10, 11]


def test_capacity_bound_is_reached():
    """Every expert with one pair more than a multiple of m: E*(m-1) padding."""
    E, m = 8, 5
    idx = np.arange(E, dtype=np.int32).reshape(E, 1)   # T = E tokens, K = 1
    lay = O.layout(idx, E, 2, m)
    assert lay.expert_offset[-1] == lay.R == E + E * (m - 1)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("scale", [False, True])
def test_padded_dispatch_compacts_to_unpadded(dtype, scale):
    rng = np.random.default_rng(11 + scale)
    T, K, E, P, m = 45, 4, 16, 4, 8
    idx = routing(rng, T, K, E, False)
    x = rows(rng, T, 24, dtype)
    w = rng.random((T, K)).astype(np.float32)
    check_padded_dispatch(O.layout, O.dispatch, idx, E, P, m, x, dtype, w, scale)
    check_padded_dispatch(O.layout, O.dispatch, idx, E, P, m, x, dtype, None, False)
    S = O.send(O.layout(idx, E, P, m), x)
    expand = lambda lay, x_, dt, w_, sc: O.expand(lay, O.send(lay, x_), dt, w_, sc)
    check_padded_dispatch(O.layout, expand, idx, E, P, m, x, dtype, w, scale)
    assert np.array_equal(S, O.send(O.layout(idx, E, P, 1), x))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_readers_never_touch_padding(dtype):
    """NaN in every padding row changes no result of a call that reads receive rows."""
    rng = np.random.default_rng(21)
    T, K, E, P, m = 38, 3, 12, 4, 8
    idx = routing(rng, T, K, E, True)
    lay, un = O.layout(idx, E, P, m), O.layout(idx, E, P, 1)
    w = rng.random((T, K)).astype(np.float32)
    y_un = rows(rng, T * K, 16, dtype)
    x = rows(rng, T, 16, dtype)
    g = rows(rng, T, 16, dtype)
    y = nan_padded(lay, un, y_un, dtype)
    for wt in (None, w):
        assert np.array_equal(O.combine(lay, y, dtype, wt), O.combine(un, y_un, dtype, wt))
        assert np.array_equal(O.dispatch_bwd(lay, y, dtype, wt)[0], O.dispatch_bwd(un, y_un, dtype, wt)[0])
        assert np.array_equal(O.combine_partitions(lay, O.reduce_partitions(lay, y, dtype, wt), dtype),
                              O.combine_partitions(un, O.reduce_partitions(un, y_un, dtype, wt), dtype))
    assert np.array_equal(O.dispatch_bwd(lay, y, dtype, w, x)[1], O.dispatch_bwd(un, y_un, dtype, w, x)[1])
    gy, gw = O.combine_bwd(lay, g, dtype, w, y)
    gyu, gwu = O.combine_bwd(un, g, dtype, w, y_un)
    assert np.array_equal(gw, gwu)
    assert np.array_equal(gy[lay.recv_pos.ravel()], gyu[un.recv_pos.ravel()])
    assert np.all(gy[pad_rows_by_loop(lay)] == 0)


# -------------------------------------------------------------- mutants -----

def layout_floor(idx, E, P, m=1):
    """Segments rounded down instead of up."""
    lay = O.layout(idx, E, P, 1)
    n = lay.num_tokens_per_expert.astype(np.int64)
    off = np.concatenate([[0], np.cumsum(n // m * m)]).astype(np.int32)
    shift = (off[:-1] - lay.expert_offset[:-1])
    e = np.asarray(idx)
    pos = lay.recv_pos + shift[e]
    return O.Layout(**{**lay.__dict__, "expert_offset": off, "recv_pos": pos.astype(np.int32),
                       "pad_multiple": m})


def layout_pad_at_front(idx, E, P, m=1):
    """Padding placed before the pairs of each segment instead of after."""
    lay = O.layout(idx, E, P, m)
    n = lay.num_tokens_per_expert.astype(np.int64)
    seg = np.diff(lay.expert_offset.astype(np.int64))
    e = np.asarray(idx)
    pos = lay.recv_pos + (seg - n)[e]
    rt = np.full(lay.R, -1, np.int32)
    rk = np.full(lay.R, -1, np.int32)
    rt[pos.ravel()] = np.repeat(np.arange(lay.T), lay.K)
    rk[pos.ravel()] = np.tile(np.arange(lay.K), lay.T)
    return O.Layout(**{**lay.__dict__, "recv_pos": pos.astype(np.int32), "recv_token": rt, "recv_k": rk})


def dispatch_no_zero_fill(lay, x, dtype, w=None, scale=False):
    recv, sc = O.dispatch(lay, x, dtype, w, scale)
    recv[lay.padding_rows()] = x[0] if len(x) else 0      # stale rows left behind
    return recv, sc


def test_mutants_fail_their_pins():
    rng = np.random.default_rng(8)
    T, K, E, P, m = 30, 3, 8, 4, 4
    idx = routing(rng, T, K, E, False)
    with pytest.raises(AssertionError):
        check_padded_layout(layout_floor, idx, E, P, m)
    with pytest.raises(AssertionError):
        check_padded_layout(layout_pad_at_front, idx, E, P, m)
    x = rows(rng, T, 8, "f32") + np.float32(1.0)
    with pytest.raises(AssertionError):
        check_padded_dispatch(O.layout, dispatch_no_zero_fill, idx, E, P, m, x, "f32", None, False)
