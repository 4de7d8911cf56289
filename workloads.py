"""Seeded synthetic inputs for the MoE layout / dispatch / combine path.

This module only draws inputs: token rows, router scores, top-k routings and
upstream gradients.  It holds none of the arithmetic of the layout, dispatch
or combine steps, and it is the one module that both the CPU oracle side and
the HIP side of the tests (and the benchmark) read their inputs from.

Routing shapes follow the MoE layers the pages discuss:

* a tiny fp32 layer (8 experts, top-2) used for quick parity checks;
* a Qwen3-30B-A3B-shaped layer (T=4096, H=2048, 128 experts, top-8);
  the pages benchmark this model family at EP8/EP16 ("Avoid collective token
  preparation for AutoEP DeepEP", section "Performance");
* two skewed variants of that layer (a Zipf-like expert popularity with one
  expert forced empty), standing in for the skewed real-SFT routing that the
  DeepEP transport PR replays ("Add an opt-in DeepEP transport ...", section
  "Why");
* a DeepSeek-V3-shaped layer (T=4096, H=7168, 256 experts, top-8, sigmoid
  scores, group-limited to 4 of 8 rank groups); its buffer sizes are the ones
  the torchtitan issue "[MoE] Apply router scores before W2 projection"
  computes in its "Motivation" section;
* a DiffusionGemma-shaped layer (T=8192, H=2816, 128 experts, top-8, scores
  absorbed before W2); H=2816 is the row width in the shapes printed by
  "perf(dllm): use the DeepEP dispatcher in the DiffusionGemma recipes".

No public dataset is read: the real routing traces, HellaSwag and Tulu-3 runs
on the pages are not available, and these synthetic routings stand in for the
routing *shape* only.

Every random stream comes from ``numpy.random.Generator(PCG64)`` seeded with
``SeedSequence([config_id, seed, step, pass, stream])``.  Router arithmetic
(softmax, sigmoid, group scores, normalisation) is done in float64 and cast
to float32 once.  bf16 tensors are drawn in float32 and rounded to bf16 by
torch's CPU conversion; they are returned as raw ``uint16`` bit patterns.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

__all__ = [
    "LayerConfig",
    "CONFIGS",
    "get_config",
    "rng_for",
    "routing",
    "normal_rows",
    "LayerInputs",
    "layer_inputs",
]

# stream ids inside one (config, seed, step, pass) seed sequence
_S_LOGITS, _S_X, _S_G, _S_Y, _S_GRECV, _S_PERM = range(6)


@dataclass(frozen=True)
class LayerConfig:
    name: str
    cid: int            # numeric id mixed into the seed
    T: int              # tokens on this GPU
    H: int              # hidden size (row width in elements)
    dtype: str          # "f32" or "bf16"
    E: int              # experts
    P: int              # virtual EP partitions (ranks)
    K: int              # top-k
    router: str         # "softmax" | "sigmoid_grouped"
    renormalize: bool   # weights scaled to sum to 1 over the top-k
    absorbed: bool      # scores applied in dispatch, combine is a plain sum
    skew: float = 0.0   # logit offset coefficient for Zipf-like popularity
    empty_expert: int = -1  # expert forced to receive no token (-1: none)
    n_groups: int = 0   # rank groups for group-limited routing
    topk_groups: int = 0

    @property
    def R(self) -> int:
        return self.T * self.K

    @property
    def esize(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def with_(self, **kw) -> "LayerConfig":
        return replace(self, **kw)


CONFIGS = {
    c.name: c
    for c in [
        LayerConfig("tiny", 1, T=256, H=128, dtype="f32", E=8, P=2, K=2,
                    router="softmax", renormalize=True, absorbed=False),
        LayerConfig("qwen3_30b_a3b", 2, T=4096, H=2048, dtype="bf16", E=128, P=8, K=8,
                    router="softmax", renormalize=True, absorbed=False),
        # Literal reading of the skew constant: c = 2.0.
        LayerConfig("skewed_literal", 3, T=4096, H=2048, dtype="bf16", E=128, P=8, K=8,
                    router="softmax", renormalize=True, absorbed=False,
                    skew=2.0, empty_expert=127),
        # Calibrated reading: c = 0.22 gives the hottest expert ~25% of tokens.
        LayerConfig("skewed_calibrated", 33, T=4096, H=2048, dtype="bf16", E=128, P=8, K=8,
                    router="softmax", renormalize=True, absorbed=False,
                    skew=0.22, empty_expert=127),
        LayerConfig("deepseek_v3", 4, T=4096, H=7168, dtype="bf16", E=256, P=64, K=8,
                    router="sigmoid_grouped", renormalize=True, absorbed=False,
                    n_groups=8, topk_groups=4),
        LayerConfig("diffusion_gemma", 5, T=8192, H=2816, dtype="bf16", E=128, P=8, K=8,
                    router="softmax", renormalize=False, absorbed=True),
    ]
}


def get_config(name: str, **overrides) -> LayerConfig:
    c = CONFIGS[name]
    return c.with_(**overrides) if overrides else c


def rng_for(cfg: LayerConfig, seed: int, step: int = 0, pss: int = 0, stream: int = 0):
    ss = np.random.SeedSequence([cfg.cid, seed, step, pss, stream])
    return np.random.Generator(np.random.PCG64(ss))


def _softmax64(logits: np.ndarray) -> np.ndarray:
    m = np.max(logits, axis=1, keepdims=True)
    z = np.exp(logits - m)
    return z / np.sum(z, axis=1, keepdims=True)


def _topk_stable(scores: np.ndarray, k: int) -> np.ndarray:
    # descending score; ties go to the lower expert id
    return np.argsort(-scores, axis=1, kind="stable")[:, :k]


def routing(cfg: LayerConfig, seed: int = 0, step: int = 0, pss: int = 0,
            idx_dtype=np.int32):
    """Top-k router decision for one layer: ``(topk_idx[T,K], topk_weights[T,K])``."""
    T, E, K = cfg.T, cfg.E, cfg.K
    rng = rng_for(cfg, seed, step, pss, _S_LOGITS)
    logits = rng.standard_normal((T, E))  # float64
    if cfg.router == "softmax":
        if cfg.skew:
            prng = rng_for(cfg, seed, 0, 0, _S_PERM)  # popularity fixed per seed
            rank_e = prng.permutation(E) + 1          # 1-based popularity rank
            logits = logits + cfg.skew * np.log(1.0 / rank_e)[None, :]
        if cfg.empty_expert >= 0:
            logits[:, cfg.empty_expert] = -np.inf
        scores = _softmax64(logits)
        idx = _topk_stable(scores, K)
        w = np.take_along_axis(scores, idx, axis=1)
    elif cfg.router == "sigmoid_grouped":
        scores = 1.0 / (1.0 + np.exp(-logits))
        G = cfg.n_groups
        per_group = E // G
        grouped = scores.reshape(T, G, per_group)
        top2 = -np.sort(-grouped, axis=2)[:, :, :2]
        gscore = top2.sum(axis=2)                              # [T,G]
        keep = _topk_stable(gscore, cfg.topk_groups)           # [T,topk_groups]
        gmask = np.zeros((T, G), dtype=bool)
        np.put_along_axis(gmask, keep, True, axis=1)
        masked = np.where(np.repeat(gmask, per_group, axis=1), scores, -np.inf)
        idx = _topk_stable(masked, K)
        w = np.take_along_axis(scores, idx, axis=1)
    else:
        raise ValueError(cfg.router)
    if cfg.renormalize:
        w = w / np.sum(w, axis=1, keepdims=True)
    return idx.astype(idx_dtype), w.astype(np.float32)


def _to_bf16_bits(a32: np.ndarray) -> np.ndarray:
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def normal_rows(cfg: LayerConfig, rows: int, stream: int, seed: int = 0,
                step: int = 0, pss: int = 0) -> np.ndarray:
    """``rows x H`` N(0,1) draw: float32 for f32 layers, bf16 bits (uint16) otherwise."""
    rng = rng_for(cfg, seed, step, pss, stream)
    a = rng.standard_normal((rows, cfg.H), dtype=np.float32)
    return a if cfg.dtype == "f32" else _to_bf16_bits(a)


@dataclass
class LayerInputs:
    cfg: LayerConfig
    topk_idx: np.ndarray       # [T,K] int32/int64
    topk_weights: np.ndarray   # [T,K] float32
    x: np.ndarray              # [T,H] tokens
    y: np.ndarray              # [R,H] expert outputs in the receive layout
    g: np.ndarray              # [T,H] gradient of the combine output
    grad_recv: np.ndarray      # [R,H] gradient of the dispatch output


def layer_inputs(cfg: LayerConfig, seed: int = 0, step: int = 0, pss: int = 0,
                 idx_dtype=np.int32, with_rows: bool = True) -> LayerInputs:
    idx, w = routing(cfg, seed, step, pss, idx_dtype)
    if not with_rows:
        empty = np.zeros((0, cfg.H), np.float32)
        return LayerInputs(cfg, idx, w, empty, empty, empty, empty)
    return LayerInputs(
        cfg, idx, w,
        x=normal_rows(cfg, cfg.T, _S_X, seed, step, pss),
        y=normal_rows(cfg, cfg.R, _S_Y, seed, step, pss),
        g=normal_rows(cfg, cfg.T, _S_G, seed, step, pss),
        grad_recv=normal_rows(cfg, cfg.R, _S_GRECV, seed, step, pss),
    )
