"""The oracle's dispatch, combine and backward passes, pinned to dense algebra,
scatter-add, exact identities and float32 error bounds."""
import numpy as np
import pytest

import workloads as W
from oracle import moe_oracle as O

import pins

CASES = [  # (T, K, E, P, H, dtype)
    (12, 3, 8, 2, 16, "f32"),
    (10, 2, 8, 4, 32, "bf16"),
    (9, 8, 8, 8, 24, "bf16"),
    (7, 1, 4, 1, 8, "f32"),
    (11, 4, 12, 6, 16, "bf16"),
]


def make(T, K, E, H, dtype, seed):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.choice(E, size=K, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, K)).astype(np.float32)
    def rows(n):
        a = rng.standard_normal((n, H)).astype(np.float32)
        return O.f32_to_bf16(a) if dtype == "bf16" else a
    return idx, w, rows(T), rows(T * K)


@pytest.mark.parametrize("T,K,E,P,H,dtype", CASES)
@pytest.mark.parametrize("seed", [0, 1])
def test_dispatch_dense(T, K, E, P, H, dtype, seed):
    idx, w, x, _ = make(T, K, E, H, dtype, seed)
    pins.check_dispatch_dense(O.layout, O.dispatch, idx, E, P, x, dtype, w)


@pytest.mark.parametrize("T,K,E,P,H,dtype", CASES)
@pytest.mark.parametrize("weighted", [True, False])
def test_combine_dense_and_scatter(T, K, E, P, H, dtype, weighted):
    idx, w, _, y = make(T, K, E, H, dtype, 3)
    ww = w if weighted else None
    pins.check_combine_dense(O.layout, O.combine, idx, E, P, y, dtype, ww)
    pins.check_combine_scatter(O.layout, O.combine, idx, E, P, y, dtype, ww)


@pytest.mark.parametrize("T,K,E,P,H,dtype", CASES)
def test_adjoint_identities_exact(T, K, E, P, H, dtype):
    rng = np.random.default_rng(5)
    idx = np.stack([rng.choice(E, size=K, replace=False) for _ in range(T)]).astype(np.int32)
    V = 4 if dtype == "f32" else 8
    pins.check_adjoints(O.layout, O.dispatch, O.combine, O.combine_bwd, O.dispatch_bwd,
                        idx, E, P, max(H, V), dtype)


def test_adjoint_wide_rows():
    # rows long enough that the canonical dot runs several rounds of 64 chunks
    rng = np.random.default_rng(6)
    idx = np.stack([rng.choice(8, size=2, replace=False) for _ in range(5)]).astype(np.int32)
    for dtype in ("f32", "bf16"):
        pins.check_adjoints(O.layout, O.dispatch, O.combine, O.combine_bwd, O.dispatch_bwd,
                            idx, 8, 2, 2 * 64 * 8 + 24, dtype)


@pytest.mark.parametrize("name", ["tiny", "qwen3_30b_a3b", "deepseek_v3", "diffusion_gemma"])
def test_k_times_x_on_config_shapes(name):
    # combine(dispatch(x)) with unit weights == K*x exactly (K*x needs <= 4 extra
    # bits for K <= 8 in bf16, and x + x is exact in f32 for K = 2).
    cfg = W.get_config(name)
    cfg = cfg.with_(T=min(cfg.T, 512))
    inp = W.layer_inputs(cfg, seed=0)
    pins.check_k_times_x(O.layout, O.dispatch, O.combine, inp.topk_idx, cfg.E, cfg.P,
                         inp.x, cfg.dtype)


@pytest.mark.parametrize("name", ["tiny", "qwen3_30b_a3b", "deepseek_v3"])
def test_unit_sum_weights_return_x(name):
    # renormalised weights sum to 1: combine(dispatch(x), w) ~= x
    cfg = W.get_config(name).with_(T=256)
    inp = W.layer_inputs(cfg, seed=0)
    lay = O.layout(inp.topk_idx, cfg.E, cfg.P)
    recv, _ = O.dispatch(lay, inp.x, cfg.dtype)
    out = pins.f64(O.combine(lay, recv, cfg.dtype, inp.topk_weights), cfg.dtype)
    x = pins.f64(inp.x, cfg.dtype)
    tol = (2 * cfg.K + 2) * pins.U32 + (pins.UBF if cfg.dtype == "bf16" else 0)
    assert np.all(np.abs(out - x) <= tol * np.abs(x) + 1e-30)


def test_scaled_dispatch_rounds_product_once():
    # bf16(f32(x) * s): compare with torch's bf16 rounding of the same float32 product
    import torch
    rng = np.random.default_rng(7)
    T, K, E, H = 6, 2, 4, 16
    idx = np.stack([rng.choice(E, size=K, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, K)).astype(np.float32)
    x = O.f32_to_bf16(rng.standard_normal((T, H)).astype(np.float32))
    lay = O.layout(idx, E, 2)
    recv, scores = O.dispatch(lay, x, "bf16", w, True)
    xf = torch.from_numpy(O.bf16_to_f32(x))
    for t in range(T):
        for k in range(K):
            ref = (xf[t] * float(w[t, k])).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            # torch multiplies by a python float in float32 here (one rounding)
            assert np.array_equal(recv[lay.recv_pos[t, k]], ref)
            assert scores[lay.recv_pos[t, k]] == w[t, k]


def test_plain_backward_copies_bits():
    rng = np.random.default_rng(8)
    idx = np.array([[0, 3], [2, 1]], np.int32)
    g = O.f32_to_bf16(rng.standard_normal((2, 8)).astype(np.float32))
    lay = O.layout(idx, 4, 2)
    gy, gw = O.combine_bwd(lay, g, "bf16")
    assert gw is None
    for t in range(2):
        for k in range(2):
            assert np.array_equal(gy[lay.recv_pos[t, k]], g[t])


def test_empty_batch_rows():
    lay = O.layout(np.zeros((0, 2), np.int32), 4, 2)
    x = np.zeros((0, 8), np.float32)
    recv, sc = O.dispatch(lay, x, "f32", np.zeros((0, 2), np.float32))
    assert recv.shape == (0, 8) and sc.shape == (0,)
    assert O.combine(lay, recv, "f32").shape == (0, 8)
