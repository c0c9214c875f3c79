"""Autograd wrappers of dispatch and combine for training.

The backward of dispatch is combine and the backward of combine is dispatch
(stakiran github-trend-summarizer, "DeepEP 要約", section 3), so each
Function's backward is one of the library's backward calls on the forward's
handle:

    recv, handle = dispatch(x, topk_idx, topk_weights, E, P)   # BF16 rows
    out = combine(y, handle, topk_weights)                     # y: expert outputs

dispatch's backward is ep_dispatch_backward (the unit-weight combine of the
received rows' gradients); combine's backward is ep_combine_backward
(weight-scaled rows of grad_out, and the weight gradient when topk_weights
requires grad).  Receive rows that no pair maps to get a zero gradient.
Only argument marshalling happens here; every step runs in the HIP kernels.
"""
from __future__ import annotations

import torch

from . import combine as _combine
from . import combine_backward as _combine_backward
from . import dispatch as _dispatch
from . import dispatch_backward as _dispatch_backward
from . import get_dispatch_layout as _get_dispatch_layout


class _Routing:
    """The layout of one dispatch; `handle` is set once dispatch has run."""

    def __init__(self, layout):
        self.layout = layout
        self.handle = None


class _Dispatch(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, topk_weights, routing, capacity_rows):
        w = topk_weights.detach().contiguous() if topk_weights is not None else None
        recv, _, handle = _dispatch(x.detach().contiguous(), w, routing.layout, False, capacity_rows)
        routing.handle = handle
        ctx.handle = handle
        return recv

    @staticmethod
    def backward(ctx, grad_recv):
        return _dispatch_backward(grad_recv.contiguous(), ctx.handle), None, None, None


def _unmapped_rows_zeroed(y, handle):
    """A gradient buffer shaped like y whose rows that no pair maps to are
    zero (the combine backward writes the others).  In a dense layout whose
    pair count the host has read (handle_recv_counts, which a grouped GEMM
    needs anyway), those rows are exactly [min(N, capacity), rows); otherwise
    every row is zeroed first."""
    c = handle.c
    dense = c.static_cap == 0 and c.expert_alignment <= 1
    if not dense or handle.num_recv is None:
        return torch.zeros_like(y, memory_format=torch.contiguous_format)
    grad_y = torch.empty_like(y, memory_format=torch.contiguous_format)
    grad_y[min(handle.num_recv, c.capacity_rows):].zero_()
    return grad_y


class _Combine(torch.autograd.Function):
    @staticmethod
    def forward(ctx, y, topk_weights, handle):
        w = topk_weights.detach().contiguous() if topk_weights is not None else None
        out = _combine(y.detach().contiguous(), handle, w)
        ctx.handle = handle
        ctx.save_for_backward(y, topk_weights)
        return out

    @staticmethod
    def backward(ctx, grad_out):
        y, w = ctx.saved_tensors
        want_w = w is not None and ctx.needs_input_grad[1]
        grad_y = _unmapped_rows_zeroed(y, ctx.handle)
        gy, gw = _combine_backward(grad_out.contiguous(), ctx.handle,
                                   y=y.detach().contiguous() if want_w else None,
                                   topk_weights=w.detach().contiguous() if w is not None else None,
                                   grad_y=grad_y)
        return gy, (gw if want_w else None), None


def dispatch(x, topk_idx, topk_weights, num_experts: int, num_partitions: int,
             capacity_rows=None):
    """BF16 dispatch with a gradient for x.  Returns (recv [capacity, H] bf16,
    handle); ep.handle_recv_counts(handle) gives the per-expert counts."""
    routing = _Routing(_get_dispatch_layout(topk_idx, num_experts, num_partitions))
    recv = _Dispatch.apply(x, topk_weights, routing, capacity_rows)
    return recv, routing.handle


def combine(y, handle, topk_weights=None):
    """Combine with gradients for y and, when it requires grad, topk_weights
    (None: the weights dispatch copied, as constants)."""
    return _Combine.apply(y, topk_weights, handle)
