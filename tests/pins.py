"""Independent checks that pin the CPU oracle to something other than itself.

Each ``check_*`` takes the oracle function under test as an argument and
raises ``AssertionError`` on a mismatch, so the same checks run against the
real oracle (must pass) and against oracle copies with a planted mistake
(must fail; see ``test_oracle_mutants.py``).

The references used here are different algorithms from the oracle's:

* layout: pure-Python loops that scan the routing once per expert (a counting
  sort by hand) instead of a library stable argsort;
* dispatch / combine: a dense 0/1 routing matrix built from that brute-force
  layout, applied in float64 (dispatch is exact; combine is held to a
  float32 rounding-error bound), and a scatter-add route for the float32 sum;
* backward passes: adjoint identities on inputs where every float32 and bf16
  operation is exact, so the identities must hold with equality;
* the canonical dot: exact integer dot products, an error bound against the
  exact sum, and hand-derived results on crafted inputs that tell the lane
  order apart from other orders.
"""
from __future__ import annotations

import math

import numpy as np

U32 = 2.0 ** -24          # float32 unit roundoff
UBF = 2.0 ** -8           # bfloat16 unit roundoff


# ---------------------------------------------------------------- layout ----

def brute_layout(idx, E, P):
    """Layout by explicit loops (no sort, no cumsum)."""
    idx = [[int(v) for v in row] for row in np.asarray(idx)]
    T = len(idx)
    K = len(idx[0]) if T else np.asarray(idx).shape[1] if np.asarray(idx).ndim == 2 else 0
    epr = E // P
    counts = [0] * E
    for t in range(T):
        for k in range(K):
            counts[idx[t][k]] += 1
    in_rank = [[0] * P for _ in range(T)]
    for t in range(T):
        for k in range(K):
            in_rank[t][idx[t][k] // epr] = 1
    per_rank = [sum(in_rank[t][r] for t in range(T)) for r in range(P)]
    eoff = [0]
    for e in range(E):
        eoff.append(eoff[-1] + counts[e])
    roff = [eoff[r * epr] for r in range(P + 1)]
    soff = [0]
    for r in range(P):
        soff.append(soff[-1] + per_rank[r])
    slot = [[-1] * P for _ in range(T)]
    for r in range(P):
        c = 0
        for t in range(T):
            if in_rank[t][r]:
                slot[t][r] = c
                c += 1
    R = T * K
    pos = [[-1] * K for _ in range(T)]
    rtok = [-1] * R
    rk = [-1] * R
    for e in range(E):
        p = eoff[e]
        for t in range(T):
            for k in range(K):
                if idx[t][k] == e:
                    pos[t][k] = p
                    rtok[p] = t
                    rk[p] = k
                    p += 1
    a = lambda v, dt=np.int32: np.array(v, dtype=dt)
    return dict(
        num_tokens_per_expert=a(counts), num_tokens_per_rank=a(per_rank),
        is_token_in_rank=a(in_rank, np.uint8).reshape(T, P),
        expert_offset=a(eoff), rank_offset=a(roff), send_offset=a(soff),
        token_slot=a(slot).reshape(T, P), recv_pos=a(pos).reshape(T, K),
        recv_token=a(rtok), recv_k=a(rk),
    )


LAYOUT_FIELDS = ("num_tokens_per_expert", "num_tokens_per_rank", "is_token_in_rank",
                 "expert_offset", "rank_offset", "send_offset", "token_slot",
                 "recv_pos", "recv_token", "recv_k")


def check_layout_brute(layout_fn, idx, E, P):
    lay = layout_fn(idx, E, P)
    ref = brute_layout(idx, E, P)
    for f in LAYOUT_FIELDS:
        got = np.asarray(getattr(lay, f))
        assert got.shape == ref[f].shape, (f, got.shape, ref[f].shape)
        assert np.array_equal(got, ref[f]), f


def check_layout_invariants(lay, idx):
    """Properties any correct layout has, checked without a second layout."""
    idx = np.asarray(idx).astype(np.int64)
    T, K = idx.shape
    E, P = lay.E, lay.P
    epr = E // P
    R = T * K
    cnt = np.asarray(lay.num_tokens_per_expert, np.int64)
    assert cnt.sum() == R                                    # every pair routed once
    pos = np.asarray(lay.recv_pos, np.int64)
    assert np.array_equal(np.sort(pos.ravel()), np.arange(R))  # bijection onto [0,R)
    eoff = np.asarray(lay.expert_offset, np.int64)
    assert eoff[0] == 0 and eoff[-1] == R and np.all(np.diff(eoff) == cnt)
    # each position inside its expert's segment
    assert np.all(pos >= eoff[idx]) and np.all(pos < eoff[idx + 1])
    # inverse maps
    rt = np.asarray(lay.recv_token, np.int64)
    rk = np.asarray(lay.recv_k, np.int64)
    assert np.array_equal(rt[pos], np.repeat(np.arange(T), K).reshape(T, K))
    assert np.array_equal(rk[pos], np.tile(np.arange(K), T).reshape(T, K))
    # stable: inside one expert, rows go by increasing (t, k)
    seg_e = np.repeat(np.arange(E), cnt)
    key = rt * K + rk
    same = seg_e[1:] == seg_e[:-1]
    assert np.all(key[1:][same] > key[:-1][same])
    # partitions
    roff = np.asarray(lay.rank_offset, np.int64)
    assert np.array_equal(roff, eoff[np.arange(P + 1) * epr])
    inr = np.asarray(lay.is_token_in_rank, np.int64)
    for r in range(P):
        hit = np.any(idx // epr == r, axis=1)
        assert np.array_equal(inr[:, r], hit.astype(np.int64))
    ntr = np.asarray(lay.num_tokens_per_rank, np.int64)
    assert np.array_equal(ntr, inr.sum(axis=0))
    n_send = ntr.sum()
    assert T <= n_send <= T * min(K, P) or T == 0             # dedup bounds
    soff = np.asarray(lay.send_offset, np.int64)
    assert soff[0] == 0 and np.array_equal(np.diff(soff), ntr)
    slot = np.asarray(lay.token_slot, np.int64)
    for r in range(P):
        s = slot[:, r]
        assert np.all((s == -1) == (inr[:, r] == 0))
        assert np.array_equal(s[inr[:, r] == 1], np.arange(ntr[r]))


# ----------------------------------------------------- rows: dense algebra --

def dense_route(ref, T, K):
    """[R, T] 0/1 matrix D with D[row of (t,k), t] = 1, from the brute layout."""
    R = T * K
    D = np.zeros((R, T))
    for t in range(T):
        for k in range(K):
            D[ref["recv_pos"][t, k], t] = 1.0
    return D


def f64(a, dtype):
    a = np.asarray(a)
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def check_dispatch_dense(layout_fn, dispatch_fn, idx, E, P, x, dtype, w=None):
    T, K = np.asarray(idx).shape
    ref = brute_layout(idx, E, P)
    D = dense_route(ref, T, K)
    recv, scores = dispatch_fn(layout_fn(idx, E, P), x, dtype, w, False)
    assert np.array_equal(f64(recv, dtype), D @ f64(x, dtype))
    if w is not None:
        expect = np.zeros(T * K)
        for t in range(T):
            for k in range(K):
                expect[ref["recv_pos"][t, k]] = w[t, k]
        assert np.array_equal(scores.astype(np.float64), expect)


def check_combine_dense(layout_fn, combine_fn, idx, E, P, y, dtype, w=None):
    """combine == Dᵀ diag(w) y up to float32 summation error (+ bf16 output rounding)."""
    T, K = np.asarray(idx).shape
    ref = brute_layout(idx, E, P)
    C = np.zeros((T, T * K))
    for t in range(T):
        for k in range(K):
            C[t, ref["recv_pos"][t, k]] = 1.0 if w is None else float(w[t, k])
    y64 = f64(y, dtype)
    exact = C @ y64
    mag = np.abs(C) @ np.abs(y64)
    out = f64(combine_fn(layout_fn(idx, E, P), y, dtype, w), dtype)
    sum_err = 2 * K * U32 * mag
    bound = sum_err + (UBF if dtype == "bf16" else 0.0) * (np.abs(exact) + sum_err) + 1e-30
    err = np.abs(out - exact)
    assert np.all(err <= bound), float(np.max(err / bound))


def check_combine_scatter(layout_fn, combine_fn, idx, E, P, y, dtype, w=None):
    """float32 equality with a scatter-add route: np.add.at over pairs in (t,k) order."""
    from oracle import moe_oracle as O   # only for the dtype conversions

    T, K = np.asarray(idx).shape
    ref = brute_layout(idx, E, P)
    yf = O.to_f32(y, dtype)
    acc = np.zeros((T, yf.shape[1]), np.float32)
    tok = np.repeat(np.arange(T), K)
    rows = yf[ref["recv_pos"].reshape(-1)]
    if w is not None:
        rows = np.asarray(w, np.float32).reshape(-1, 1) * rows
    np.add.at(acc, tok, rows)
    out = combine_fn(layout_fn(idx, E, P), y, dtype, w)
    assert np.array_equal(np.asarray(out), O.from_f32(acc, dtype))


# ------------------------------------------- rows: exact adjoint identities --

def exact_inputs(rng, T, H, K, dtype):
    """Small-integer rows and power-of-two weights: every op below is exact.

    Products |w*y| <= 2*4, sums of K<=8 such terms stay within 8 significant
    bits at step 0.5, so even bf16 outputs are exact.
    """
    def rows(n):
        a = rng.integers(-4, 5, size=(n, H)).astype(np.float32)
        if dtype == "bf16":
            return (a.view(np.uint32) >> 16).astype(np.uint16)
        return a
    w = rng.choice(np.array([0.5, 1.0, 2.0], np.float32), size=(T, K))
    return rows(T), rows(T * K), rows(T), rows(T * K), w


def check_adjoints(layout_fn, dispatch_fn, combine_fn, combine_bwd_fn, dispatch_bwd_fn,
                   idx, E, P, H, dtype, seed=0):
    T, K = np.asarray(idx).shape
    rng = np.random.default_rng(seed)
    x, y, g, G, w = exact_inputs(rng, T, H, K, dtype)
    lay = layout_fn(idx, E, P)
    ip = lambda a, b: float(np.sum(f64(a, dtype) * f64(b, dtype)))

    # unscaled dispatch and its backward
    recv, _ = dispatch_fn(lay, x, dtype, None, False)
    gx, _ = dispatch_bwd_fn(lay, G, dtype, None, None)
    assert ip(recv, G) == ip(x, gx)
    # scaled dispatch: linear in x and in w
    recv_s, _ = dispatch_fn(lay, x, dtype, w, True)
    gx_s, gs = dispatch_bwd_fn(lay, G, dtype, w, x)
    assert ip(recv_s, G) == ip(x, gx_s)
    assert ip(recv_s, G) == float(np.sum(w.astype(np.float64) * gs.astype(np.float64)))
    # weighted combine and its backward
    out = combine_fn(lay, y, dtype, w)
    gy, gw = combine_bwd_fn(lay, g, dtype, w, y)
    assert ip(out, g) == ip(y, gy)
    assert ip(out, g) == float(np.sum(w.astype(np.float64) * gw.astype(np.float64)))
    # plain combine
    out_p = combine_fn(lay, y, dtype, None)
    gy_p, gw_p = combine_bwd_fn(lay, g, dtype, None, None)
    assert gw_p is None
    assert ip(out_p, g) == ip(y, gy_p)


def check_k_times_x(layout_fn, dispatch_fn, combine_fn, idx, E, P, x, dtype):
    """combine(dispatch(x)) with unit weights equals K*x exactly."""
    T, K = np.asarray(idx).shape
    lay = layout_fn(idx, E, P)
    recv, _ = dispatch_fn(lay, x, dtype, None, False)
    out = combine_fn(lay, recv, dtype, None)
    assert np.array_equal(f64(out, dtype), K * f64(x, dtype))


# ---------------------------------------------------------- canonical dot ---

def check_dot_integer(dot_fn, dtype, n=7, H=None, seed=0):
    """Integer-valued rows: all partial sums are exact, so the result is the exact dot."""
    rng = np.random.default_rng(seed)
    V = 4 if dtype == "f32" else 8
    H = H or V * 200
    a = rng.integers(-8, 9, size=(n, H)).astype(np.float32)
    b = rng.integers(-8, 9, size=(n, H)).astype(np.float32)
    exact = np.array([sum(int(p) * int(q) for p, q in zip(a[i], b[i])) for i in range(n)])
    if dtype == "bf16":
        a = (a.view(np.uint32) >> 16).astype(np.uint16)
        b = (b.view(np.uint32) >> 16).astype(np.uint16)
    got = dot_fn(a, b, dtype)
    assert np.array_equal(got.astype(np.float64), exact.astype(np.float64))


def check_dot_bound(dot_fn, dtype, n=5, H=2048, seed=1):
    """Random rows: |dot32 - exact| <= gamma_H * sum|a*b| (Higham, any order)."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((n, H)).astype(np.float32)
    b = rng.standard_normal((n, H)).astype(np.float32)
    if dtype == "bf16":
        a = (a.view(np.uint32) >> 16).astype(np.uint16)
        b = (b.view(np.uint32) >> 16).astype(np.uint16)
    got = dot_fn(a, b, dtype).astype(np.float64)
    A, B = f64(a, dtype), f64(b, dtype)
    for i in range(n):
        exact = math.fsum((A[i] * B[i]).tolist())        # products exact in f64
        mag = float(np.sum(np.abs(A[i] * B[i])))
        gamma = (H + 1) * U32 / (1 - (H + 1) * U32)
        assert abs(got[i] - exact) <= gamma * mag


def dot_order_cases(dtype="f32"):
    """Crafted rows whose canonical result is derived by hand.

    Rows have 256 chunks of V elements (V = 4 for f32, 8 for bf16), so 4
    segments of 64 chunks.  ``at(j, i)`` is element i of chunk j.  b is all
    ones, so every product is the a value itself.  All values are exact in
    bf16.  Write B = 2^24: B + 1 is a float32 tie and rounds to B (even).

    Case A (fold order inside a segment): B at (0,0), -B at (1,0), 1 at
    (32,0) and 1 at (33,0), all in segment 0.  Fold s=32: partial 0 = B + 1
    -> B, partial 1 = -B + 1 = -(B - 1) exactly; s=16..2 add zeros; s=1:
    B - (B - 1) = 1.  Result 1.0.  Left to right gives B - B + 1 + 1 = 2.0;
    folding neighbours first (s = 1, ..., 32) gives 0 + 2 = 2.0; segments of
    32 chunks give 0 + 2 = 2.0.

    Case B (segments are folded on their own, then added): B at (0,0) in
    segment 0, 1 at (64,0) and 1 at (65,0) in segment 1.  Segment values B
    and 2; result B + 2 exactly.  Carrying one partial per lane across
    segments (chunks 0 and 64 on partial 0) absorbs each 1 into B: B.  Left
    to right also gives B.

    Case C (segment values added in sequence from +0.0): 1 at (0,0), B at
    (64,0), 1 at (128,0), 1 at (192,0): segment values 1, B, 1, 1.
    Sequentially: 1 + B -> B, + 1 -> B, + 1 -> B.  Result B.  A pairwise tree
    gives (1 + B -> B) + (1 + 1) = B + 2; adding in reverse order gives
    2 + B = B + 2, + 1 -> B + 4 (tie to even).

    Case D (elements of a chunk are added in order): B at (0,0), 1 at (0,1)
    and 1 at (0,2).  Chunk partial: B + 1 -> B, + 1 -> B.  Result B.  Adding
    the chunk's elements last to first gives 1 + 1 + B = B + 2.
    """
    V = 4 if dtype == "f32" else 8
    H = 256 * V
    a = np.zeros((4, H), np.float32)
    b = np.ones((4, H), np.float32)
    at = lambda j, i: j * V + i
    big = 2.0 ** 24
    a[0, at(0, 0)], a[0, at(1, 0)], a[0, at(32, 0)], a[0, at(33, 0)] = big, -big, 1.0, 1.0
    a[1, at(0, 0)], a[1, at(64, 0)], a[1, at(65, 0)] = big, 1.0, 1.0
    a[2, at(0, 0)], a[2, at(64, 0)], a[2, at(128, 0)], a[2, at(192, 0)] = 1.0, big, 1.0, 1.0
    a[3, at(0, 0)], a[3, at(0, 1)], a[3, at(0, 2)] = big, 1.0, 1.0
    expect = np.array([1.0, big + 2.0, big, big], np.float32)
    if dtype == "bf16":
        a = (a.view(np.uint32) >> 16).astype(np.uint16)
        b = (b.view(np.uint32) >> 16).astype(np.uint16)
    return a, b, expect


def check_dot_order(dot_fn, dtype="f32"):
    a, b, expect = dot_order_cases(dtype)
    got = dot_fn(a, b, dtype)
    assert np.array_equal(got, expect), got
