"""Seeded synthetic inputs for anchor attention (numpy only).

This module is shared by the HIP path's tests/benchmark and by the oracle's tests.
It holds no arithmetic of the method itself: it only draws random tensors, applies
the workload's value structure (scales, noise, "sink" tokens) and rounds to the
storage dtype.

Shapes follow the library's layout: Q, K, V are [B, h, n, d] and the anchors U are
[h, m, d] (learnable parameters of each head, shared over the batch).

Recipe (per workload; numpy PCG64 ``default_rng(seed)``):
  1. draw fp32 standard normals in the order Q, K, V, U, each in its full shape;
  2. apply the workload's structure in fp32 (Q scale; U from K rows plus noise;
     sink-token scaling), drawing any extra random numbers after step 1;
  3. round once, round-to-nearest-even, to the storage dtype (bf16 or fp32).
The returned float32 arrays hold the exact stored values; for bf16 workloads the
raw uint16 bit patterns are returned as well (numpy has no bf16 dtype).

The workloads mirror AnchorFormer's ViT settings (AnchorFormer pages: ImageNet
ViT token grids, the anchor-count sweet spot near 30) and two larger stress shapes;
real images and trained weights are not available, so these seeded draws stand in
for them.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    h: int
    n: int
    m: int
    d: int
    dtype: str            # "fp32" or "bf16"
    seed: int
    q_scale: float = 1.0  # Q multiplied by this (peaked softmax rows)
    u_from_k_rows: bool = False   # U = m distinct rows of K[0, head] + noise
    u_noise_std: float = 0.0
    sink_frac: float = 0.0        # fraction of tokens whose Q, K, V rows are scaled
    sink_scale: float = 1.0
    description: str = ""

    @property
    def slices(self) -> int:
        return self.B * self.h

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "fp32" else 2

    def algorithmic_bytes(self) -> int:
        """Q and V read once, H written once, U read once per head."""
        es = self.elem_bytes
        return 3 * self.B * self.h * self.n * self.d * es + self.h * self.m * self.d * es

    def algorithmic_flops(self) -> int:
        """2nmd each for the logits, A^T V and A W, per (batch, head) slice."""
        return 6 * self.B * self.h * self.n * self.m * self.d


WORKLOADS: dict[str, Workload] = {w.name: w for w in [
    Workload("tiny_fp32", B=1, h=1, n=64, m=8, d=32, dtype="fp32", seed=1001,
             description="tiny fp32 slice; checked against the explicit two-step chain"),
    Workload("vit_s16_224", B=64, h=6, n=196, m=30, d=64, dtype="bf16", seed=1002,
             description="ViT-S/16 at 224px: 14x14 patch grid, 6 heads, 30 anchors"),
    Workload("vit_b16_384", B=32, h=12, n=576, m=64, d=64, dtype="bf16", seed=1003,
             q_scale=2.0, description="ViT-B/16 at 384px: 24x24 grid, 12 heads, Q x2"),
    Workload("dense_64x64", B=8, h=8, n=4096, m=128, d=64, dtype="bf16", seed=1004,
             u_from_k_rows=True, u_noise_std=0.1,
             description="dense-prediction 64x64 map; anchors = K rows + N(0, 0.1^2) noise"),
    Workload("long_16k_fp32", B=2, h=16, n=16384, m=256, d=64, dtype="fp32", seed=1005,
             sink_frac=0.01, sink_scale=10.0,
             description="long sequence, fp32; 1% of tokens x10 (attention-sink-like)"),
    Workload("long_16k_bf16", B=2, h=16, n=16384, m=256, d=64, dtype="bf16", seed=1005,
             sink_frac=0.01, sink_scale=10.0,
             description="long sequence, bf16; 1% of tokens x10 (attention-sink-like)"),
]}

HEADLINE = "vit_s16_224"


def bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Inputs:
    workload: Workload
    Q: np.ndarray          # float32 exact stored values [B,h,n,d]
    K: np.ndarray
    V: np.ndarray
    U: np.ndarray          # [h,m,d]
    bits: dict = field(default_factory=dict)   # bf16 only: name -> uint16 array

    def stored(self, name: str) -> np.ndarray:
        """The array as stored on the device: uint16 bits (bf16) or float32."""
        if self.workload.dtype == "bf16":
            return self.bits[name]
        return getattr(self, name)


def _store(x: np.ndarray, dtype: str):
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "fp32":
        return x, None
    bits = bf16_bits_rne(x)
    return bf16_bits_to_f32(bits), bits


def make_inputs(w: Workload | str, seed: int | None = None, with_k: bool = True,
                shape: dict | None = None) -> Inputs:
    """Draw one input set for workload ``w`` (optionally overriding seed or sizes).

    ``shape`` may override any of B, h, n, m, d (used for small parity cases that
    keep a workload's value structure)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    if shape:
        w = Workload(**{**w.__dict__, **shape})
    if seed is None:
        seed = w.seed
    rng = np.random.default_rng(seed)
    B, h, n, m, d = w.B, w.h, w.n, w.m, w.d
    Q = rng.standard_normal((B, h, n, d), dtype=np.float32)
    K = rng.standard_normal((B, h, n, d), dtype=np.float32) if (with_k or w.u_from_k_rows) else None
    V = rng.standard_normal((B, h, n, d), dtype=np.float32)
    U = rng.standard_normal((h, m, d), dtype=np.float32)
    if w.q_scale != 1.0:
        Q *= np.float32(w.q_scale)
    if w.u_from_k_rows:
        if m > n:
            raise ValueError("anchors drawn from K rows need m <= n")
        for head in range(h):
            idx = rng.choice(n, size=m, replace=False)
            U[head] = K[0, head, idx, :]
        U += np.float32(w.u_noise_std) * rng.standard_normal((h, m, d), dtype=np.float32)
    if w.sink_frac > 0.0:
        ns = int(round(w.sink_frac * n))
        for b in range(B):
            idx = rng.choice(n, size=ns, replace=False)
            for arr in (Q, K, V):
                if arr is not None:
                    arr[b, :, idx, :] *= np.float32(w.sink_scale)
    out = Inputs(workload=w, Q=None, K=None, V=None, U=None)
    for name, arr in (("Q", Q), ("K", K), ("V", V), ("U", U)):
        if arr is None:
            continue
        vals, bits = _store(arr, w.dtype)
        setattr(out, name, vals)
        if bits is not None:
            out.bits[name] = bits
    return out


def random_case(seed: int, B: int, h: int, n: int, m: int, d: int, dtype: str = "fp32",
                q_scale: float = 1.0) -> Inputs:
    """Plain N(0,1) inputs of an arbitrary shape (edge-case and sweep tests)."""
    w = Workload(f"case_{B}x{h}x{n}x{m}x{d}_{dtype}", B=B, h=h, n=n, m=m, d=d, dtype=dtype,
                 seed=seed, q_scale=q_scale)
    return make_inputs(w, with_k=False)


def make_upstream_grad(x: Inputs, seed: int) -> tuple[np.ndarray, np.ndarray | None]:
    """A seeded upstream gradient dL/dH of the shape of ``x.Q`` (N(0,1), fp32 draws in
    one call of ``default_rng(seed)``), rounded once to the workload's storage dtype.

    Returns (stored values as float32, uint16 bf16 bit patterns or None for fp32)."""
    rng = np.random.default_rng(seed)
    g = rng.standard_normal(x.Q.shape, dtype=np.float32)
    return _store(g, x.workload.dtype)


def make_landmarks(B: int, n: int, s: int, seed: int) -> np.ndarray:
    """Landmark token indices for Nystrom attention, int32 [B, s]: token 0 (the class
    token, always a landmark) and s - 1 distinct other tokens per batch element, drawn
    with ``default_rng(seed)``; the heads of a batch element share them.  A seeded stand-in
    for farthest-point sampling on token features."""
    if not 1 <= s <= n:
        raise ValueError("need 1 <= s <= n landmarks")
    rng = np.random.default_rng(seed)
    rows = [np.concatenate([[0], rng.choice(np.arange(1, n), size=s - 1, replace=False)])
            for _ in range(B)]
    return np.ascontiguousarray(np.stack(rows).astype(np.int32))


@dataclass
class BlockInputs:
    """Inputs of the attention block around the layer; float32 stored values plus bf16
    bit patterns (name -> uint16 array) for bf16."""
    B: int
    n: int
    h: int
    m: int
    d: int
    dtype: str
    X: np.ndarray
    Wqv: np.ndarray
    bqv: np.ndarray
    U: np.ndarray
    Wo: np.ndarray
    bo: np.ndarray
    bits: dict = field(default_factory=dict)


def make_block_inputs(B: int, n: int, h: int, m: int, d: int, seed: int,
                      dtype: str = "bf16") -> BlockInputs:
    """Seeded block inputs (numpy PCG64 ``default_rng(seed)``, drawn in this order):
    X [B, n, C] ~ N(0, 1); Wqv [C, 2C] ~ N(0, 1/C) (so Q and V entries have unit
    variance); bqv [2C] ~ N(0, 0.1^2); U [h, m, d] ~ N(0, 1); Wo [C, C] ~ N(0, 1/C);
    bo [C] ~ N(0, 0.1^2); each rounded once to the storage dtype."""
    rng = np.random.default_rng(seed)
    C = h * d
    sc = np.float32(1.0 / np.sqrt(C))
    raw = {
        "X": rng.standard_normal((B, n, C), dtype=np.float32),
        "Wqv": rng.standard_normal((C, 2 * C), dtype=np.float32) * sc,
        "bqv": rng.standard_normal((2 * C,), dtype=np.float32) * np.float32(0.1),
        "U": rng.standard_normal((h, m, d), dtype=np.float32),
        "Wo": rng.standard_normal((C, C), dtype=np.float32) * sc,
        "bo": rng.standard_normal((C,), dtype=np.float32) * np.float32(0.1),
    }
    vals, bits = {}, {}
    for k, a in raw.items():
        v, b = _store(a, dtype)
        vals[k] = v
        if b is not None:
            bits[k] = b
    return BlockInputs(B=B, n=n, h=h, m=m, d=d, dtype=dtype, bits=bits, **vals)
