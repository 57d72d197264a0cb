"""MI355X-native (gfx950) AnchorFormer anchor attention.

The compute lives in a C-ABI HIP library (``csrc/``, header ``include/anchor_attn.h``);
``anchor_attn`` is its thin Python binding, ``autograd`` wraps forward and backward as a
differentiable torch function, and ``inputs`` is the seeded workload generator.  Importing the package does not load the GPU library; the first call
through the binding does, and raises if it is missing.
"""
from .anchor_attn import forward, AnchorAttention, library_path  # noqa: F401


def anchor_attention(Q, U, V):
    """Differentiable anchor attention (gradients for Q, U and V through the library)."""
    from .autograd import anchor_attention as _f
    return _f(Q, U, V)


__all__ = ["forward", "AnchorAttention", "library_path", "anchor_attention"]
