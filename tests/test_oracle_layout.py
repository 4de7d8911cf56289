"""The oracle's layout, pinned to brute force and to invariants."""
import numpy as np
import pytest

import workloads as W
from oracle import moe_oracle as O

from pins import brute_layout, check_layout_brute, check_layout_invariants


def rand_idx(rng, T, K, E, distinct=True):
    if distinct:
        return np.stack([rng.choice(E, size=K, replace=False) for _ in range(T)]).reshape(T, K).astype(np.int32)
    return rng.integers(0, E, size=(T, K)).astype(np.int32)


TINY = [  # (T, K, E, P)
    (1, 1, 1, 1), (1, 3, 8, 4), (12, 3, 8, 2), (12, 2, 8, 4), (9, 3, 6, 3),
    (7, 8, 8, 8), (11, 4, 8, 1), (10, 2, 4, 4), (5, 1, 8, 2), (12, 3, 12, 6),
]


@pytest.mark.parametrize("T,K,E,P", TINY)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_brute_force_random(T, K, E, P, seed):
    rng = np.random.default_rng(seed)
    idx = rand_idx(rng, T, K, E)
    check_layout_brute(O.layout, idx, E, P)
    check_layout_invariants(O.layout(idx, E, P), idx)


@pytest.mark.parametrize("seed", [0, 1])
def test_brute_force_duplicates(seed):
    # duplicate expert ids inside one token are ordered by (t, k)
    rng = np.random.default_rng(seed)
    idx = rand_idx(rng, 12, 3, 4, distinct=False)
    check_layout_brute(O.layout, idx, 4, 2)
    check_layout_invariants(O.layout(idx, 4, 2), idx)


def edge_cases():
    yield "all_on_one_expert", np.full((9, 1), 5, np.int32), 8, 4
    yield "empty_first_expert", np.array([[1, 2], [3, 1], [2, 7]], np.int32), 8, 2
    yield "empty_middle_expert", np.array([[0, 1], [1, 7], [0, 7]], np.int32), 8, 2
    yield "empty_last_expert", np.array([[0, 1], [3, 2], [6, 5]], np.int32), 8, 2
    yield "empty_partition", np.array([[0, 1], [2, 3], [1, 0]], np.int32), 8, 4
    yield "K_equals_E", np.array([[3, 1, 0, 2], [0, 1, 2, 3]], np.int32), 4, 2
    yield "P_equals_E", np.array([[0, 5], [5, 7], [6, 0]], np.int32), 8, 8
    yield "P_is_1", np.array([[0, 5], [5, 7], [6, 0]], np.int32), 8, 1
    yield "T_is_1", np.array([[7, 0, 3]], np.int32), 8, 4
    yield "int64_ids", np.array([[7, 0], [3, 4]], np.int64), 8, 2


@pytest.mark.parametrize("name,idx,E,P", list(edge_cases()), ids=[c[0] for c in edge_cases()])
def test_edge_cases(name, idx, E, P):
    check_layout_brute(O.layout, idx, E, P)
    check_layout_invariants(O.layout(idx, E, P), idx)


def test_empty_batch():
    idx = np.zeros((0, 3), np.int32)
    lay = O.layout(idx, 8, 2)
    assert lay.recv_pos.shape == (0, 3) and lay.recv_token.shape == (0,)
    assert np.array_equal(lay.expert_offset, np.zeros(9, np.int32))
    assert np.array_equal(lay.send_offset, np.zeros(3, np.int32))


def test_empty_expert_offsets_repeat():
    idx = np.array([[0, 1], [3, 2], [6, 5]], np.int32)  # experts 4 and 7 empty
    lay = O.layout(idx, 8, 2)
    assert lay.expert_offset[4] == lay.expert_offset[5]
    assert lay.expert_offset[7] == lay.expert_offset[8] == 6


def test_rejects_bad_input():
    with pytest.raises(ValueError):
        O.layout(np.array([[0, 8]]), 8, 2)
    with pytest.raises(ValueError):
        O.layout(np.array([[0, -1]]), 8, 2)
    with pytest.raises(ValueError):
        O.layout(np.array([[0, 1]]), 6, 4)


@pytest.mark.parametrize("name", list(W.CONFIGS))
def test_invariants_on_config_routings(name):
    cfg = W.get_config(name)
    idx, _ = W.routing(cfg, seed=0)
    lay = O.layout(idx, cfg.E, cfg.P)
    check_layout_invariants(lay, idx)
    if cfg.empty_expert >= 0:
        e = cfg.empty_expert
        assert lay.num_tokens_per_expert[e] == 0
        assert lay.expert_offset[e] == lay.expert_offset[e + 1] == cfg.R


def test_brute_force_on_a_slice_of_each_config():
    # brute force is O(E*T*K) in Python: use 40 tokens of each routing
    for name in W.CONFIGS:
        cfg = W.get_config(name)
        idx, _ = W.routing(cfg, seed=1)
        check_layout_brute(O.layout, idx[:40], cfg.E, cfg.P)


def test_replay_gives_identical_layout():
    cfg = W.get_config("diffusion_gemma")
    idx, _ = W.routing(cfg, seed=0)
    a, b = O.layout(idx, cfg.E, cfg.P), O.layout(idx.copy(), cfg.E, cfg.P)
    for f in ("recv_pos", "recv_token", "recv_k", "token_slot", "expert_offset"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
