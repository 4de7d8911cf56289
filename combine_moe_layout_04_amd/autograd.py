"""Autograd wrappers: one handle shared by a Dispatch and its paired Combine.

Each backward pass runs the opposite row movement on the routing the forward
used: the dispatch's backward sums receive-row gradients back to tokens, and
the combine's backward spreads the output gradient to the receive rows
("Add an opt-in DeepEP transport for the AutoEP expert all-to-all", section
"Why").  Both return the router-weight gradient, without which the gate
would stop learning (the review fix on that page).  Nothing here computes:
every step is a library call.

The C handle keeps only its latest layout.  A backward pass whose handle was
laid out again after its forward (for example a per-layer handle reused by a
later forward pass) raises instead of using the newer routing.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import api


class StaleLayoutError(RuntimeError):
    """The handle was laid out again between a forward pass and its backward."""


def _same_layout(ctx, what):
    if ctx.handle.generation != ctx.generation:
        raise StaleLayoutError(
            f"{what} backward: the handle holds layout {ctx.handle.generation}, but the forward pass "
            f"used layout {ctx.generation}; give each forward pass that takes a backward its own handle, "
            "or replay the layout before the backward")


class _Dispatch(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, topk_weights, handle, scale_rows):
        recv, scores = api.moe_dispatch(handle, x, topk_weights, scale_rows=scale_rows,
                                        recv_scores=topk_weights is not None)
        ctx.handle = handle
        ctx.generation = handle.generation
        ctx.scale_rows = bool(scale_rows)
        ctx.save_for_backward(x if scale_rows else None, topk_weights if scale_rows else None)
        if scores is not None:
            # per-row scores are returned for a downstream consumer; their
            # gradient reaches the router through the scaling (grad_s) or the
            # combine's weights (grad_w), not through this output
            ctx.mark_non_differentiable(scores)
        return recv, scores

    @staticmethod
    def backward(ctx, grad_recv, _grad_scores):
        _same_layout(ctx, "dispatch")
        x, w = ctx.saved_tensors
        want_s = ctx.scale_rows and ctx.needs_input_grad[1]
        grad_x, grad_s = api.moe_dispatch_bwd(ctx.handle, grad_recv.contiguous(),
                                              w if ctx.scale_rows else None,
                                              x if want_s else None, grad_s=want_s)
        return grad_x, grad_s, None, None


class _Combine(torch.autograd.Function):
    @staticmethod
    def forward(ctx, y, topk_weights, handle):
        out = api.moe_combine(handle, y, topk_weights)
        ctx.handle = handle
        ctx.generation = handle.generation
        ctx.weighted = topk_weights is not None
        ctx.save_for_backward(y if ctx.weighted else None, topk_weights)
        return out

    @staticmethod
    def backward(ctx, grad_out):
        _same_layout(ctx, "combine")
        y, w = ctx.saved_tensors
        want_w = ctx.weighted and ctx.needs_input_grad[1]
        grad_y, grad_w = api.moe_combine_bwd(ctx.handle, grad_out.contiguous(), w,
                                             y if want_w else None, grad_w=want_w)
        return grad_y, grad_w, None


def dispatch(x: torch.Tensor, topk_weights: Optional[torch.Tensor], handle: api.Handle,
             scale_rows: bool = False):
    """Differentiable dispatch; returns (recv, recv_scores or None)."""
    return _Dispatch.apply(x, topk_weights, handle, scale_rows)


def combine(y: torch.Tensor, topk_weights: Optional[torch.Tensor], handle: api.Handle) -> torch.Tensor:
    """Differentiable combine (plain sum when topk_weights is None)."""
    return _Combine.apply(y, topk_weights, handle)
