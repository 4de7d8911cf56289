"""Values the pages print, checked against the oracle's buffer shapes.

The only numbers the pages give for this path are buffer sizes (the
torchtitan issue's DeepSeek V3 memory estimate) and a capacity; the
numerics of dispatch and combine are pinned by the other oracle tests.
"""
import json
import os

import numpy as np

import workloads as W
from oracle import moe_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden", "page_sizes.json")
MiB = 1 << 20
GiB = 1 << 30


def load():
    with open(GOLD) as f:
        return json.load(f)


def test_deepseek_layer_buffer_sizes_from_the_oracle():
    g = load()
    cfg = W.get_config("deepseek_v3")
    assert (cfg.T, cfg.K, cfg.H, cfg.esize) == (g["T"], g["top_k"], g["D"], g["bytes_per_elem"])
    inp = W.layer_inputs(cfg, seed=0, with_rows=False)
    x = np.zeros((cfg.T, cfg.H), np.uint16)
    lay = O.layout(inp.topk_idx, cfg.E, cfg.P)
    recv, _ = O.dispatch(lay, x, "bf16")
    assert recv.nbytes / MiB == g["w2_output_MiB_per_layer"]
    out = O.combine(lay, recv[:, :8], "bf16")          # narrow rows: shape only
    assert out.shape[0] * cfg.H * cfg.esize / MiB == g["combine_output_MiB_per_layer"]
    L = g["moe_layers"]
    assert round(recv.nbytes * L / GiB, 1) == g["w2_output_GiB_all_layers"]
    assert round(out.shape[0] * cfg.H * cfg.esize * L / GiB, 2) == g["combine_output_GiB_all_layers"]
    # The page adds its two rounded figures (25.4 + 3.17); the exact total is
    # 28.55 GiB, which the page's 28.6 reaches only through that rounding.
    w2 = round(recv.nbytes * L / GiB, 1)
    comb = round(out.shape[0] * cfg.H * cfg.esize * L / GiB, 2)
    assert round(w2 + comb, 1) == g["total_GiB_per_gpu"]


def test_capacity_is_microbatch_product():
    g = load()
    assert g["microbatch"][0] * g["microbatch"][1] == g["num_max_tokens_per_rank"]
    # one receive row per routed pair: R = T * top_k
    assert O.recv_rows(g["T"], g["top_k"]) == g["T"] * g["top_k"]
