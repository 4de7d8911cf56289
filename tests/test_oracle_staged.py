"""Pins for the oracle's staged exchange (a deduplicated send buffer per
destination partition, receiver-side expansion, and the two-level combine).

References that are not the oracle's own code:
* explicit Python loops over (token, partition) and (token, k) pairs, with
  float32 scalar arithmetic, for the send buffer, send_token and both levels
  of the combine;
* the single-stage dispatch (itself pinned by brute force and dense algebra):
  a staged dispatch copies the same bits to the same rows;
* exact integer arithmetic, where every order of summation gives the same
  result, and the fp64 adjoint identities.
Planted mistakes (in oracle copies, on the CPU) must fail these pins.
"""
import numpy as np
import pytest

from oracle import moe_oracle as O


SHAPES = [  # T, K, E, P, duplicates allowed
    (1, 1, 1, 1, False), (9, 2, 4, 2, False), (33, 3, 12, 4, False), (40, 4, 8, 8, False),
    (25, 4, 6, 3, True), (60, 8, 32, 8, False), (17, 5, 20, 1, False),
]


def routing(rng, T, K, E, dup):
    if dup:
        return rng.integers(0, E, size=(T, K)).astype(np.int32)
    return np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)


def rows(rng, n, H, dtype, integer=False):
    a = (rng.integers(-4, 5, size=(n, H)) if integer else rng.standard_normal((n, H))).astype(np.float32)
    return a if dtype == "f32" else O.f32_to_bf16(a)


def f32(a, dtype):
    return O.to_f32(a, dtype)


# ----------------------------------------------------------- brute force ----

def brute_send(idx, E, P, x):
    """Loops over tokens and partitions, counting slots by hand."""
    idx = np.asarray(idx)
    T, K = idx.shape
    epr = E // P
    member = [[any(int(idx[t, k]) // epr == r for k in range(K)) for r in range(P)] for t in range(T)]
    counts = [sum(member[t][r] for t in range(T)) for r in range(P)]
    start = [sum(counts[:r]) for r in range(P)]
    S = np.zeros((sum(counts), x.shape[1]), dtype=x.dtype)
    tok = [0] * sum(counts)
    for r in range(P):
        slot = 0
        for t in range(T):
            if member[t][r]:
                S[start[r] + slot] = x[t]
                tok[start[r] + slot] = t
                slot += 1
    return S, np.array(tok, np.int32)


def brute_two_level(idx, E, P, y_rows_of_pairs, dtype, w=None):
    """Two-level combine by scalar float32 loops.  y_rows_of_pairs[t][k] is
    the receive row of pair (t,k) as float32."""
    idx = np.asarray(idx)
    T, K = idx.shape
    epr = E // P
    H = y_rows_of_pairs.shape[2]
    one = np.float32
    out = np.zeros((T, H), dtype=np.float32)
    Q = {}
    for t in range(T):
        for r in range(P):
            ks = [k for k in range(K) if int(idx[t, k]) // epr == r]
            if not ks:
                continue
            part = np.zeros(H, dtype=np.float32)
            for h in range(H):
                acc = one(0.0)
                for k in ks:
                    v = y_rows_of_pairs[t, k, h]
                    term = one(one(w[t, k]) * v) if w is not None else v
                    acc = one(acc + term)
                part[h] = acc
            Q[(t, r)] = O.to_f32(O.from_f32(part, dtype), dtype)   # rounded to the row type
    for t in range(T):
        for h in range(H):
            acc = one(0.0)
            for r in range(P):
                if (t, r) in Q:
                    acc = one(acc + Q[(t, r)][h])
            out[t, h] = acc
    return O.from_f32(out, dtype), Q


# ----------------------------------------------------------------- pins -----

def check_send(layout_fn, send_fn, idx, E, P, x):
    lay = layout_fn(idx, E, P)
    S_ref, tok_ref = brute_send(idx, E, P, x)
    S = send_fn(lay, x)
    assert S.shape == S_ref.shape
    assert np.array_equal(S, S_ref)
    assert np.array_equal(lay.send_token, tok_ref)


def check_expand_is_dispatch(layout_fn, send_fn, expand_fn, idx, E, P, x, dtype, w):
    lay = layout_fn(idx, E, P)
    for scale in (False, True):
        r1, s1 = expand_fn(lay, send_fn(lay, x), dtype, w, scale)
        r2, s2 = O.dispatch(lay, x, dtype, w, scale)
        assert np.array_equal(r1, r2)
        assert np.array_equal(s1, s2)


def check_two_level(layout_fn, reduce_fn, combine_fn, idx, E, P, y, dtype, w):
    lay = layout_fn(idx, E, P)
    yp = f32(y, dtype)[lay.recv_pos]                    # [T,K,H]
    out_ref, Q_ref = brute_two_level(idx, E, P, yp, dtype, w)
    Q = reduce_fn(lay, y, dtype, w)
    for (t, r), q in Q_ref.items():
        assert np.array_equal(f32(Q[lay.send_offset[r] + lay.token_slot[t, r]], dtype), q), (t, r)
    assert np.array_equal(combine_fn(lay, Q, dtype), out_ref)


@pytest.mark.parametrize("T,K,E,P,dup", SHAPES)
def test_send_buffer_brute_force(T, K, E, P, dup):
    rng = np.random.default_rng(T * 31 + K)
    idx = routing(rng, T, K, E, dup)
    check_send(O.layout, O.send, idx, E, P, rows(rng, T, 8, "bf16"))


@pytest.mark.parametrize("T,K,E,P,dup", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_expand_of_send_is_dispatch(T, K, E, P, dup, dtype):
    rng = np.random.default_rng(T * 7 + E)
    idx = routing(rng, T, K, E, dup)
    w = rng.random((T, K)).astype(np.float32)
    check_expand_is_dispatch(O.layout, O.send, O.expand, idx, E, P, rows(rng, T, 16, dtype), dtype, w)


@pytest.mark.parametrize("T,K,E,P,dup", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("weighted", [False, True])
def test_two_level_combine_brute_force(T, K, E, P, dup, dtype, weighted):
    rng = np.random.default_rng(T * 13 + P)
    idx = routing(rng, T, K, E, dup)
    w = rng.random((T, K)).astype(np.float32) if weighted else None
    check_two_level(O.layout, O.reduce_partitions, O.combine_partitions, idx, E, P,
                    rows(rng, T * K, 8, dtype), dtype, w)


def test_two_level_order_is_observable():
    """Crafted rows where the two levels give a different float32 result
    from k order.  Token 0 routes k = 0, 1, 2 to experts 0, 1, 0 (E = P = 2:
    partitions 0, 1, 0) with values 1, 2^24, 1.  k order: 1 + 2^24 is a tie
    and rounds to 2^24, + 1 rounds to 2^24 again.  Two levels: partition 0
    sums 1 + 1 = 2, partition 1 holds 2^24, and the source adds 2 + 2^24 =
    2^24 + 2 exactly.  So the two-level result is 2^24 + 2, the single-level
    one 2^24."""
    idx = np.array([[0, 1, 0]], np.int32)  # a duplicate expert id is allowed (ordered by k)
    lay = O.layout(idx, 2, 2)
    y = np.zeros((3, 4), np.float32)
    y[lay.recv_pos[0, 0], 0] = 1.0
    y[lay.recv_pos[0, 1], 0] = 2.0 ** 24
    y[lay.recv_pos[0, 2], 0] = 1.0
    two = O.combine_partitions(lay, O.reduce_partitions(lay, y, "f32"), "f32")
    one = O.combine(lay, y, "f32")
    assert two[0, 0] == 2.0 ** 24 + 2.0
    assert one[0, 0] == 2.0 ** 24


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_integer_rows_match_single_level_and_dense(dtype):
    """Small integers: every partial sum is exact, so the two-level combine
    equals the single-level one and the dense fp64 sum."""
    rng = np.random.default_rng(5)
    T, K, E, P = 50, 6, 24, 6
    idx = routing(rng, T, K, E, False)
    lay = O.layout(idx, E, P)
    y = rows(rng, T * K, 24, dtype, integer=True)
    two = O.combine_partitions(lay, O.reduce_partitions(lay, y, dtype), dtype)
    assert np.array_equal(two, O.combine(lay, y, dtype))
    dense = f32(y, dtype).astype(np.float64)[lay.recv_pos].sum(axis=1)
    assert np.array_equal(f32(two, dtype).astype(np.float64), dense)


def test_staged_adjoint_exact():
    """<expand(send(x)), G> == <x, combine_partitions(reduce_partitions(G))>
    on small integers (all arithmetic exact)."""
    rng = np.random.default_rng(9)
    T, K, E, P = 40, 4, 16, 4
    idx = routing(rng, T, K, E, False)
    lay = O.layout(idx, E, P)
    x = rows(rng, T, 12, "f32", integer=True)
    G = rows(rng, T * K, 12, "f32", integer=True)
    lhs = np.sum(O.expand(lay, O.send(lay, x), "f32")[0].astype(np.float64) * G)
    rhs = np.sum(x.astype(np.float64) * O.combine_partitions(lay, O.reduce_partitions(lay, G, "f32"), "f32"))
    assert lhs == rhs


def test_empty_batch():
    lay = O.layout(np.zeros((0, 3), np.int32), 6, 3)
    assert lay.n_send == 0 and lay.send_token.shape == (0,)
    assert O.send(lay, np.zeros((0, 8), np.float32)).shape == (0, 8)
    Q = O.reduce_partitions(lay, np.zeros((0, 8), np.float32), "f32")
    assert O.combine_partitions(lay, Q, "f32").shape == (0, 8)


# -------------------------------------------------------------- mutants -----

def send_off_by_one(lay, x):
    S = O.send(lay, x)
    return np.roll(S, 1, axis=0)


def expand_wrong_partition(lay, S, dtype, w=None, scale=False):
    bad = O.Layout(**{**lay.__dict__, "part": (lay.part + 1) % lay.P})
    return O.expand(bad, S, dtype, w, scale)


def reduce_ignores_partition(lay, y, dtype, w=None):
    # every partition's partial sums all k (as if the dedup were ignored)
    yf = O.to_f32(y, dtype)
    full = np.zeros((lay.T, yf.shape[1]), np.float32)
    for k in range(lay.K):
        term = yf[lay.recv_pos[:, k]]
        if w is not None:
            term = np.asarray(w, np.float32)[:, k:k + 1] * term
        full = full + term
    return O.from_f32(full[lay.send_token], dtype)


def combine_partitions_descending(lay, Q, dtype):
    Qf = O.to_f32(Q, dtype)
    acc = np.zeros((lay.T, Qf.shape[1]), np.float32)
    for r in range(lay.P - 1, -1, -1):
        ts = np.nonzero(lay.is_token_in_rank[:, r])[0]
        acc[ts] = acc[ts] + Qf[lay.send_offset[r] + lay.token_slot[ts, r]]
    return O.from_f32(acc, dtype)


def test_mutants_fail_their_pins():
    rng = np.random.default_rng(3)
    T, K, E, P = 33, 3, 12, 4
    idx = routing(rng, T, K, E, False)
    x = rows(rng, T, 8, "f32")
    with pytest.raises(AssertionError):
        check_send(O.layout, send_off_by_one, idx, E, P, x)
    w = rng.random((T, K)).astype(np.float32)
    with pytest.raises(AssertionError):
        check_expand_is_dispatch(O.layout, O.send, expand_wrong_partition, idx, E, P, x, "f32", w)
    y = rows(rng, T * K, 8, "f32")
    with pytest.raises(AssertionError):
        check_two_level(O.layout, reduce_ignores_partition, O.combine_partitions, idx, E, P, y, "f32", w)
    # descending partition order: visible on rows built so that the order matters
    big = np.float32(2.0 ** 24)
    idx2 = np.array([[0, 1, 2]], np.int32)          # three partitions, one expert each
    lay2 = O.layout(idx2, 3, 3)
    y2 = np.zeros((3, 4), np.float32)
    y2[lay2.recv_pos[0, 0], 0] = 1.0
    y2[lay2.recv_pos[0, 1], 0] = 1.0
    y2[lay2.recv_pos[0, 2], 0] = big
    Q2 = O.reduce_partitions(lay2, y2, "f32")
    assert O.combine_partitions(lay2, Q2, "f32")[0, 0] == big + 2       # 1 + 1 + 2^24
    assert combine_partitions_descending(lay2, Q2, "f32")[0, 0] == big  # 2^24 + 1 -> 2^24, + 1 -> 2^24
    with pytest.raises(AssertionError):
        check_two_level(O.layout, O.reduce_partitions, combine_partitions_descending, idx2, 3, 3,
                        y2, "f32", None)
