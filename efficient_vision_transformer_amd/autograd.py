"""torch.autograd integration: anchor attention as a differentiable function, so that Q, U
(the learnable anchors) and V receive gradients in an ordinary training step.

Both directions run in the HIP library through the C ABI (anchor_attn_forward and
anchor_attn_backward); this module only hands tensors over.  The backward's domain is
the library's: bf16 with m <= 256 (m <= 128 at d = 128), fp32 with m <= 256 and d = 32 or
64; U's gradient is summed over the batch.
"""
from __future__ import annotations

import torch

from .anchor_attn import AnchorAttention, shared_context


def _context(device) -> AnchorAttention:
    # one context per (device, current stream): the backward may run on another stream
    # than the forward (autograd's own streams), and contexts must not share workspaces
    # across streams
    return shared_context(device, torch.cuda.current_stream(device))


class AnchorAttentionFunction(torch.autograd.Function):
    """H = A (Delta^-1 (A^T V)), A = rowsoftmax(Q U^T / sqrt(d)); Q, V [B, h, n, d] (views
    whose d values per token are contiguous, e.g. halves of a packed projection), U [h, m, d]
    contiguous, all on one GPU."""

    @staticmethod
    def forward(fctx, Q, U, V):
        ctx = _context(Q.device)
        H = ctx.forward(Q, U, V)
        fctx.save_for_backward(Q, U, V)
        return H

    @staticmethod
    def backward(fctx, dH):
        Q, U, V = fctx.saved_tensors
        ctx = _context(Q.device)
        if dH.stride(-1) != 1:
            dH = dH.contiguous()
        dQ, dU, dV = ctx.backward(Q, U, V, dH)
        return dQ, dU, dV


def anchor_attention(Q, U, V):
    """Differentiable anchor attention (see AnchorAttentionFunction)."""
    return AnchorAttentionFunction.apply(Q, U, V)
