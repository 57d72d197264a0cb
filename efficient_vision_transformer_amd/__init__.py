"""MI355X-native (gfx950) AnchorFormer anchor attention.

The compute lives in a C-ABI HIP library (``csrc/``, header ``include/anchor_attn.h``);
``anchor_attn`` is its thin Python binding and ``inputs`` the seeded workload
generator.  Importing the package does not load the GPU library; the first call
through the binding does, and raises if it is missing.
"""
from .anchor_attn import forward, AnchorAttention, library_path  # noqa: F401

__all__ = ["forward", "AnchorAttention", "library_path"]
