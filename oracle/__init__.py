"""fp64 CPU oracle for AnchorFormer anchor attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and its
Python binding) never imports, links or calls it, and it imports nothing from the
product package.

The arithmetic lives in ``anchor_oracle.c`` (plain C, fp64, libm ``exp``), built with
gcc into ``libanchor_oracle.so`` next to this file.  This module only marshals numpy
arrays (upcast exactly to float64) into that library.

Functions
---------
anchor_attn(Q, U, V, nthreads)      -- H for [B,h,n,d] tensors, U [h,m,d]; Eq. (12) order
anchor_slice(q, u, v)               -- one slice, returns (A, delta, W, H)
anchor_bruteforce(q, u, v)          -- one slice via the bipartite chain F = D^-1 G, F^2;
                                       returns (S_t, H)
full_attention_slice(q, k, v, rows) -- report-only softmax(QK^T/sqrt(d))V for chosen rows
anchor_backward(Q, U, V, G)         -- dQ, dU (summed over the batch), dV for dL/dH = G
anchor_block_forward(X, Wqv, bqv, U, Wo, bo)
                                    -- the attention block around the layer: numpy fp64
                                       projections (a library primitive) around anchor_attn
relu_linear_attn(Q, K, V, cmin, qscale)
                                    -- L2ViT's ReLU linear attention (numpy fp64)
nystrom_attn(Q, K, V, idx)          -- Nystrom attention with given landmark tokens
                                       (Fast Nystrom Attention page; numpy fp64)
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "anchor_oracle.c")
_DEFAULT_LIB = os.path.join(_HERE, "libanchor_oracle.so")
# ANCHOR_ORACLE_LIB names another build of anchor_oracle.c to load (the sanitizer test's)
_LIB = os.environ.get("ANCHOR_ORACLE_LIB") or _DEFAULT_LIB
_lib = None

_DBL = ctypes.POINTER(ctypes.c_double)
_LONGP = ctypes.POINTER(ctypes.c_long)
_L = ctypes.c_long


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (fp64, no fused contraction, no fast-math)."""
    if force or not os.path.exists(_DEFAULT_LIB):
        tmp = _DEFAULT_LIB + ".tmp"
        cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
               "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _DEFAULT_LIB)
    return _DEFAULT_LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        lib.oracle_anchor_slice_f64.argtypes = [_DBL, _DBL, _DBL, _L, _L, _L, _DBL, _DBL, _DBL, _DBL]
        lib.oracle_anchor_attn_f64.argtypes = [_DBL, _DBL, _DBL, _DBL, _L, _L, _L, _L, _L, ctypes.c_int]
        lib.oracle_anchor_bruteforce_f64.argtypes = [_DBL, _DBL, _DBL, _L, _L, _L, _DBL, _DBL]
        lib.oracle_full_attn_slice_f64.argtypes = [_DBL, _DBL, _DBL, _L, _L, _LONGP, _L, _DBL]
        lib.oracle_anchor_backward_slice_f64.argtypes = [_DBL, _DBL, _DBL, _DBL, _L, _L, _L,
                                                         _DBL, _DBL, _DBL]
        lib.oracle_anchor_backward_f64.argtypes = [_DBL, _DBL, _DBL, _DBL, _DBL, _DBL, _DBL,
                                                   _L, _L, _L, _L, _L, ctypes.c_int]
        for f in (lib.oracle_anchor_slice_f64, lib.oracle_anchor_attn_f64,
                  lib.oracle_anchor_bruteforce_f64, lib.oracle_full_attn_slice_f64):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    """Host threads for the batched oracle: the cores this process may use, at most 16
    (the CPU share of one GPU on a shared box)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _p(x: np.ndarray):
    return x.ctypes.data_as(_DBL)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


def anchor_slice(q, u, v):
    """One slice: q [n,d], u [m,d], v [n,d] -> (A [n,m], delta [m], W [m,d], H [n,d])."""
    q, u, v = _f64(q), _f64(u), _f64(v)
    n, d = q.shape
    m = u.shape[0]
    assert u.shape == (m, d) and v.shape == (n, d)
    A = np.zeros((n, m)); delta = np.zeros(m); W = np.zeros((m, d)); H = np.zeros((n, d))
    _check(_load().oracle_anchor_slice_f64(_p(q), _p(u), _p(v), n, m, d, _p(A), _p(delta),
                                          _p(W), _p(H)), "anchor_slice")
    return A, delta, W, H


def anchor_attn(Q, U, V, nthreads: int | None = None) -> np.ndarray:
    """Q, V [B,h,n,d]; U [h,m,d] -> H [B,h,n,d] in fp64."""
    Q, U, V = _f64(Q), _f64(U), _f64(V)
    B, h, n, d = Q.shape
    m = U.shape[1]
    assert U.shape == (h, m, d) and V.shape == Q.shape
    if nthreads is None:
        nthreads = default_threads()
    H = np.zeros_like(Q)
    _check(_load().oracle_anchor_attn_f64(_p(Q), _p(U), _p(V), _p(H), B, h, n, m, d,
                                         int(nthreads)), "anchor_attn")
    return H


def anchor_backward_slice(q, u, v, gh):
    """Gradients of one slice for dL/dH = gh -> (dq [n,d], du [m,d], dv [n,d])."""
    q, u, v, gh = _f64(q), _f64(u), _f64(v), _f64(gh)
    n, d = q.shape
    m = u.shape[0]
    assert u.shape == (m, d) and v.shape == (n, d) and gh.shape == (n, d)
    dq = np.zeros((n, d)); du = np.zeros((m, d)); dv = np.zeros((n, d))
    _check(_load().oracle_anchor_backward_slice_f64(_p(q), _p(u), _p(v), _p(gh), n, m, d,
                                                   _p(dq), _p(du), _p(dv)), "backward_slice")
    return dq, du, dv


def anchor_backward(Q, U, V, G, nthreads: int | None = None):
    """Q, V, G [B,h,n,d]; U [h,m,d] -> (dQ [B,h,n,d], dU [h,m,d] summed over the batch,
    dV [B,h,n,d]) in fp64."""
    Q, U, V, G = _f64(Q), _f64(U), _f64(V), _f64(G)
    B, h, n, d = Q.shape
    m = U.shape[1]
    assert U.shape == (h, m, d) and V.shape == Q.shape and G.shape == Q.shape
    if nthreads is None:
        nthreads = default_threads()
    dQ = np.zeros_like(Q); dV = np.zeros_like(Q); dU = np.zeros_like(U)
    _check(_load().oracle_anchor_backward_f64(_p(Q), _p(U), _p(V), _p(G), _p(dQ), _p(dU),
                                             _p(dV), B, h, n, m, d, int(nthreads)),
           "backward")
    return dQ, dU, dV


def anchor_bruteforce(q, u, v):
    """One slice through F = D^-1 G and F^2 -> (S_t [n,n], H [n,d])."""
    q, u, v = _f64(q), _f64(u), _f64(v)
    n, d = q.shape
    m = u.shape[0]
    S = np.zeros((n, n)); H = np.zeros((n, d))
    _check(_load().oracle_anchor_bruteforce_f64(_p(q), _p(u), _p(v), n, m, d, _p(S), _p(H)),
           "anchor_bruteforce")
    return S, H


def full_attention_slice(q, k, v, rows=None) -> np.ndarray:
    """Report-only: softmax(q k^T / sqrt(d)) v for the given rows (all rows if None)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    n, d = q.shape
    if rows is None:
        rows_arr, nrows, rp = None, n, None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows, rp = rows_arr.size, rows_arr.ctypes.data_as(_LONGP)
    out = np.zeros((nrows, d))
    _check(_load().oracle_full_attn_slice_f64(_p(q), _p(k), _p(v), n, d, rp, nrows, _p(out)),
           "full_attention_slice")
    return out


def anchor_block_forward(X, Wqv, bqv, U, Wo, bo) -> np.ndarray:
    """The attention block in which the layer replaces a ViT block's self-attention
    (AnchorFormer as a drop-in attention module in DeiT / LeViT backbones, Pith verdict
    page; the pages print no projections, so the plain multi-head reading): for X
    [B, n, C] with C = h*d,
        [Q | V] = X Wqv + bqv       (head j: columns j*d .. j*d + d - 1 of each half)
        H = anchor_attn per (batch, head) with U [h, m, d]
        Y = H Wo + bo               (H's columns head-major, as Q's)
    bqv or bo may be None.  fp64; the matrix products are numpy's."""
    X, Wqv, U, Wo = _f64(X), _f64(Wqv), _f64(U), _f64(Wo)
    B, n, C = X.shape
    h, m, d = U.shape
    assert h * d == C and Wqv.shape == (C, 2 * C) and Wo.shape == (C, C)
    QV = X @ Wqv
    if bqv is not None:
        QV = QV + _f64(bqv)
    Q = QV[..., :C].reshape(B, n, h, d).transpose(0, 2, 1, 3)
    V = QV[..., C:].reshape(B, n, h, d).transpose(0, 2, 1, 3)
    H = anchor_attn(np.ascontiguousarray(Q), U, np.ascontiguousarray(V))
    Y = H.transpose(0, 2, 1, 3).reshape(B, n, C) @ Wo
    if bo is not None:
        Y = Y + _f64(bo)
    return Y


def relu_linear_attn(Q, K, V, cmin: float = 100.0, qscale: float = 1.0) -> np.ndarray:
    """ReLU kernel linear attention (L2ViT page, the decomposable kernel identity of its
    Eq. (4) with phi = ReLU and the denominator clamped below at Cmin), per (batch, head)
    slice of Q, K, V [B, h, n, d]:
        S = phi(K)^T V (d x d),  z = phi(K)^T 1 (d),
        out_i = phi(qscale * q_i) S / max(phi(qscale * q_i) . z, cmin).
    qscale stands for 1/s, the page's learnable scale (initialised to sqrt(C)) read as a
    divisor of the query-key products; for qscale > 0 it only moves the clamp.  fp64."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    assert Q.shape == K.shape == V.shape and Q.ndim == 4
    phq = np.maximum(Q * float(qscale), 0.0)
    phk = np.maximum(K, 0.0)
    S = np.matmul(phk.transpose(0, 1, 3, 2), V)          # [B, h, d, d]
    z = phk.sum(axis=2)                                   # [B, h, d]
    num = np.matmul(phq, S)                               # [B, h, n, d]
    den = np.einsum("bhnd,bhd->bhn", phq, z)
    return num / np.maximum(den, float(cmin))[..., None]


def _row_softmax(x: np.ndarray) -> np.ndarray:
    e = np.exp(x - x.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def nystrom_attn(Q, K, V, idx) -> np.ndarray:
    """Nystrom attention (Fast Nystrom Attention page, key machinery: the attention matrix
    taken as the product of three row softmaxes through s landmark rows q, k of Q and K,
    the middle one inverted).  Per (batch b, head j) slice, with the landmarks the token
    rows idx[b] (s distinct indices per batch element, shared by the heads) and c = 1/sqrt(d):
        F1 = rowsoftmax(Q k^T c)   (n x s: tokens against the landmark keys)
        F2 = rowsoftmax(q k^T c)   (s x s)
        F3 = rowsoftmax(q K^T c)   (s x n: each landmark query over all tokens)
        H  = F1 (F2^-1 (F3 V)),
    the n x n product never formed.  F2^-1 is applied by a linear solve (numpy's LU with
    partial pivoting, a library primitive; equal to the pseudo-inverse when F2 is
    nonsingular).  Q, K, V [B, h, n, d]; idx [B, s] integers.  fp64."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    idx = np.asarray(idx)
    assert Q.shape == K.shape == V.shape and Q.ndim == 4
    B, h, n, d = Q.shape
    assert idx.ndim == 2 and idx.shape[0] == B
    c = 1.0 / np.sqrt(d)
    H = np.empty_like(Q)
    for b in range(B):
        ib = idx[b]
        for j in range(h):
            q, k, v = Q[b, j], K[b, j], V[b, j]
            ql, kl = q[ib], k[ib]
            F1 = _row_softmax((q @ kl.T) * c)
            F2 = _row_softmax((ql @ kl.T) * c)
            F3 = _row_softmax((ql @ k.T) * c)
            H[b, j] = F1 @ np.linalg.solve(F2, F3 @ v)
    return H
