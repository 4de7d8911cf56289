"""Gradient check of the oracle's backward passes, one input element at a time.

Each forward pass is linear in its rows and, separately, in its router
weights.  On inputs where every float32 and bfloat16 operation is exact
(small integers, power-of-two weights, short sums), a unit step in one input
element therefore changes the loss <g, f(...)> by exactly that element's
gradient.  This is a finite-difference gradcheck with no step-size error: it
checks every element of grad_x, grad_y, grad_w and grad_s, padding rows
included, so a swapped k, a gradient sent to the wrong token or row, or a
transposed operand fails.  The last test chains the passes through a
per-expert linear "expert", as a training step does, with every backward pass
replayed against the forward's layout ("Add an opt-in DeepEP transport for the
AutoEP expert all-to-all", section "Why")."""
import numpy as np
import pytest

from oracle import moe_oracle as O

import pins

CASES = [  # (T, K, E, P, pad_multiple, dtype)
    (1, 1, 4, 1, 1, "f32"),
    (5, 2, 4, 2, 1, "f32"),
    (4, 3, 6, 3, 1, "bf16"),
    (5, 2, 6, 2, 3, "bf16"),
    (3, 3, 4, 4, 2, "f32"),
]
H = 8


def values(a, dtype):
    return pins.f64(a, dtype)


def encode(v, dtype):
    """float64 values that are exact in the row type, as that type's array."""
    f = np.asarray(v, np.float64).astype(np.float32)
    assert np.array_equal(f.astype(np.float64), v)
    if dtype == "bf16":
        bits = f.view(np.uint32)
        assert np.all(bits & 0xFFFF == 0), "not exact in bfloat16"
        return (bits >> 16).astype(np.uint16)
    return f


def make(T, K, E, P, pad, dtype, seed):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.choice(E, size=K, replace=False) for _ in range(T)]).astype(np.int32)
    lay = O.layout(idx, E, P, pad)

    def rows(n):
        return rng.integers(-4, 5, size=(n, H)).astype(np.float64)

    w = rng.choice(np.array([0.5, 1.0, 2.0]), size=(T, K))
    return lay, rows(T), rows(lay.R), w, rows(T), rows(lay.R)


def bump(a, i, step=1.0):
    b = a.copy()
    b[i] += step
    return b


def row_grad(lay, gy, i):
    """The gradient of receive-row element i: rows past the last expert's
    segment (the unused tail of a worst-case-sized padded buffer) are left
    unwritten by the backward pass, and their gradient is zero."""
    return gy[i] if i[0] < lay.expert_offset[-1] else 0.0


def loss(out, g, dtype):
    return float(np.sum(values(out, dtype) * g))


@pytest.mark.parametrize("T,K,E,P,pad,dtype", CASES)
@pytest.mark.parametrize("weighted", [True, False])
def test_combine_gradients(T, K, E, P, pad, dtype, weighted):
    lay, _, y, w, g, _ = make(T, K, E, P, pad, dtype, 1)
    wt = w.astype(np.float32) if weighted else None
    f = lambda y_, w_: loss(O.combine(lay, encode(y_, dtype), dtype,
                                      None if w_ is None else w_.astype(np.float32)), g, dtype)
    gy, gw = O.combine_bwd(lay, encode(g, dtype), dtype, wt, encode(y, dtype) if weighted else None)
    gy = values(gy, dtype)
    base = f(y, w if weighted else None)
    for i in np.ndindex(y.shape):
        assert f(bump(y, i), w if weighted else None) - base == row_grad(lay, gy, i), ("grad_y", i)
    if weighted:
        for i in np.ndindex(w.shape):
            assert f(y, bump(w, i)) - base == float(gw[i]), ("grad_w", i)
    else:
        assert gw is None


@pytest.mark.parametrize("T,K,E,P,pad,dtype", CASES)
@pytest.mark.parametrize("scaled", [True, False])
def test_dispatch_gradients(T, K, E, P, pad, dtype, scaled):
    lay, x, _, w, _, G = make(T, K, E, P, pad, dtype, 2)
    f = lambda x_, w_: loss(O.dispatch(lay, encode(x_, dtype), dtype, w_.astype(np.float32),
                                       scaled)[0], G, dtype)
    gx, gs = O.dispatch_bwd(lay, encode(G, dtype), dtype, w.astype(np.float32) if scaled else None,
                            encode(x, dtype) if scaled else None)
    gx = values(gx, dtype)
    base = f(x, w)
    for i in np.ndindex(x.shape):
        assert f(bump(x, i), w) - base == gx[i], ("grad_x", i)
    if scaled:
        for i in np.ndindex(w.shape):
            assert f(x, bump(w, i)) - base == float(gs[i]), ("grad_s", i)
    else:
        assert gs is None
        for i in np.ndindex(w.shape):     # an unscaled dispatch does not depend on w
            assert f(x, bump(w, i)) == base


@pytest.mark.parametrize("T,K,E,P,pad,dtype", CASES)
def test_two_level_combine_has_the_combine_gradients(T, K, E, P, pad, dtype):
    """The staged combine computes the same function, so combine_bwd is its
    backward too: checked by stepping its own inputs."""
    lay, _, y, w, g, _ = make(T, K, E, P, pad, dtype, 3)

    def f(y_, w_):
        Q = O.reduce_partitions(lay, encode(y_, dtype), dtype, w_.astype(np.float32))
        return loss(O.combine_partitions(lay, Q, dtype), g, dtype)

    gy, gw = O.combine_bwd(lay, encode(g, dtype), dtype, w.astype(np.float32), encode(y, dtype))
    gy = values(gy, dtype)
    base = f(y, w)
    for i in np.ndindex(y.shape):
        assert f(bump(y, i), w) - base == row_grad(lay, gy, i), ("grad_y", i)
    for i in np.ndindex(w.shape):
        assert f(y, bump(w, i)) - base == float(gw[i]), ("grad_w", i)


@pytest.mark.parametrize("T,K,E,P,pad,dtype", CASES)
@pytest.mark.parametrize("absorbed", [False, True])
def test_layer_chain_gradients(T, K, E, P, pad, dtype, absorbed):
    """L(x, w) = <g, combine(c * dispatch(x, w), w)> with a per-expert scale c
    standing in for the experts.  The gradients come from the backward passes
    run in reverse order against the same layout: combine_bwd gives grad_y and
    (weighted) grad_w; the expert step scales grad_y by c; dispatch_bwd gives
    grad_x and (absorbed) grad_s."""
    lay, x, _, w, g, _ = make(T, K, E, P, pad, dtype, 4)
    if dtype == "bf16" and K == 3:
        x = np.clip(x, -2, 2)        # keeps every sum within bfloat16's 8 bits
    rng = np.random.default_rng(5)
    c_e = rng.choice(np.array([1.0, 2.0]), size=E)
    end = int(lay.expert_offset[-1])
    owner = np.repeat(np.arange(E), np.diff(lay.expert_offset))   # expert of each used receive row
    c_row = c_e[owner][:, None]

    def expert(recv):
        """Scales each expert's rows; the unused tail rows stay zero."""
        out = np.zeros((lay.R, H))
        out[:end] = values(recv[:end], dtype) * c_row
        return encode(out, dtype)

    def f(x_, w_):
        wf = w_.astype(np.float32)
        recv, _ = O.dispatch(lay, encode(x_, dtype), dtype, wf, absorbed)
        out = O.combine(lay, expert(recv), dtype, None if absorbed else wf)
        return loss(out, g, dtype)

    wf = w.astype(np.float32)
    recv, _ = O.dispatch(lay, encode(x, dtype), dtype, wf, absorbed)
    y = expert(recv)
    gy, gw = O.combine_bwd(lay, encode(g, dtype), dtype, None if absorbed else wf,
                           None if absorbed else y)
    g_recv = expert(gy)                      # the expert is symmetric: its backward scales by c
    gx, gs = O.dispatch_bwd(lay, g_recv, dtype, wf if absorbed else None,
                            encode(x, dtype) if absorbed else None)
    grad_w = gs if absorbed else gw
    gx = values(gx, dtype)
    base = f(x, w)
    for i in np.ndindex(x.shape):
        assert f(bump(x, i), w) - base == gx[i], ("grad_x", i)
    for i in np.ndindex(w.shape):
        assert f(x, bump(w, i)) - base == float(grad_w[i]), ("grad_w", i)


def test_a_planted_mistake_fails_the_check():
    """The check can tell: a grad_w with two k columns swapped is caught."""
    lay, _, y, w, g, _ = make(5, 2, 4, 2, 1, "f32", 1)
    wf = w.astype(np.float32)
    _, gw = O.combine_bwd(lay, encode(g, "f32"), "f32", wf, encode(y, "f32"))
    bad = gw[:, ::-1]
    base = loss(O.combine(lay, encode(y, "f32"), "f32", wf), g, "f32")
    steps = [loss(O.combine(lay, encode(y, "f32"), "f32", bump(w, i).astype(np.float32)), g, "f32") - base
             for i in np.ndindex(w.shape)]
    assert np.array_equal(np.array(steps).reshape(w.shape), gw)
    assert not np.array_equal(np.array(steps).reshape(w.shape), bad)
