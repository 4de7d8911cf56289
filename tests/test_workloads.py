"""The synthetic routings have the structure each layer shape calls for."""
import numpy as np
import pytest

import workloads as W


@pytest.mark.parametrize("name", list(W.CONFIGS))
def test_routing_shape_and_determinism(name):
    cfg = W.get_config(name)
    a, wa = W.routing(cfg, seed=0)
    b, wb = W.routing(cfg, seed=0)
    c, _ = W.routing(cfg, seed=1)
    assert a.shape == (cfg.T, cfg.K) and wa.dtype == np.float32
    assert np.array_equal(a, b) and np.array_equal(wa, wb)
    assert not np.array_equal(a, c)
    # distinct experts per token, ids in range
    assert np.all(np.sort(a, axis=1)[:, 1:] != np.sort(a, axis=1)[:, :-1])
    assert a.min() >= 0 and a.max() < cfg.E
    if cfg.renormalize:
        assert np.allclose(wa.sum(axis=1), 1.0, atol=1e-6)
    else:
        assert np.all(wa.sum(axis=1) < 1.0)


def test_group_limited_routing():
    cfg = W.get_config("deepseek_v3")
    idx, _ = W.routing(cfg, seed=0)
    groups = idx // (cfg.E // cfg.n_groups)       # 8 groups of 32 experts = 8 ranks each
    n_groups = np.array([len(set(r)) for r in groups.tolist()])
    assert n_groups.max() <= cfg.topk_groups
    ranks = idx // (cfg.E // cfg.P)
    assert max(len(set(r)) for r in ranks.tolist()) <= cfg.K


@pytest.mark.parametrize("name,lo,hi", [("skewed_calibrated", 0.2, 0.3), ("skewed_literal", 0.95, 1.0)])
def test_skew(name, lo, hi):
    cfg = W.get_config(name)
    idx, _ = W.routing(cfg, seed=0)
    share = max(np.mean(np.any(idx == e, axis=1)) for e in range(cfg.E))
    assert lo <= share <= hi
    assert not np.any(idx == cfg.empty_expert)


def test_rows_dtype():
    cfg = W.get_config("tiny")
    assert W.normal_rows(cfg, 3, 1).dtype == np.float32
    cfg2 = W.get_config("qwen3_30b_a3b").with_(T=4)
    r = W.normal_rows(cfg2, 3, 1)
    assert r.dtype == np.uint16 and r.shape == (3, cfg2.H)
