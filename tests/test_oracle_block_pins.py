"""Pins of the oracle's attention block (projections around anchor attention), CPU only.

The block is a reading (the pages call the layer a drop-in attention module but print no
projections): [Q | V] = X Wqv + bqv, heads of d consecutive columns, H = anchor attention
per (batch, head), Y = H Wo + bo.  Each pin fixes a different part: explicit loops through
the bipartite two-step chain, identity projections, a closed form for constant
projections, and the independence of the heads' order."""
import numpy as np
import pytest

import oracle


def _rand(seed, B, n, h, m, d):
    r = np.random.default_rng(seed)
    C = h * d
    X = r.standard_normal((B, n, C))
    Wqv = r.standard_normal((C, 2 * C)) / np.sqrt(C)
    bqv = 0.1 * r.standard_normal(2 * C)
    U = r.standard_normal((h, m, d))
    Wo = r.standard_normal((C, C)) / np.sqrt(C)
    bo = 0.1 * r.standard_normal(C)
    return X, Wqv, bqv, U, Wo, bo


def _rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


@pytest.mark.parametrize("seed", range(3))
def test_block_equals_loops_through_the_two_step_chain(seed):
    """Projections as explicit sums in Python loops, each slice through the brute-force
    S_t of F = D^-1 G (H = S_t V), the output projection as explicit sums."""
    B, n, h, m, d = 2, 5, 2, 3, 4
    X, Wqv, bqv, U, Wo, bo = _rand(seed, B, n, h, m, d)
    C = h * d
    QV = np.zeros((B, n, 2 * C))
    for b in range(B):
        for t in range(n):
            for j in range(2 * C):
                QV[b, t, j] = bqv[j] + sum(X[b, t, k] * Wqv[k, j] for k in range(C))
    Hc = np.zeros((B, n, C))
    for b in range(B):
        for j in range(h):
            q = QV[b, :, j * d:(j + 1) * d]
            v = QV[b, :, C + j * d:C + (j + 1) * d]
            _, H = oracle.anchor_bruteforce(q, U[j], v)
            Hc[b, :, j * d:(j + 1) * d] = H
    Y = np.zeros((B, n, C))
    for b in range(B):
        for t in range(n):
            for j in range(C):
                Y[b, t, j] = bo[j] + sum(Hc[b, t, k] * Wo[k, j] for k in range(C))
    got = oracle.anchor_block_forward(X, Wqv, bqv, U, Wo, bo)
    assert _rel(got, Y) <= 1e-12


def test_identity_projections_reduce_to_the_layer():
    B, n, h, m, d = 2, 17, 3, 5, 8
    X, _, _, U, _, _ = _rand(3, B, n, h, m, d)
    C = h * d
    Wqv = np.concatenate([np.eye(C), np.eye(C)], axis=1)
    got = oracle.anchor_block_forward(X, Wqv, None, U, np.eye(C), None)
    Xh = np.ascontiguousarray(X.reshape(B, n, h, d).transpose(0, 2, 1, 3))
    H = oracle.anchor_attn(Xh, U, Xh)
    assert _rel(got, H.transpose(0, 2, 1, 3).reshape(B, n, C)) <= 1e-14


def test_constant_projections_closed_form():
    """Wqv = 0: every token has the same q and v (the biases), so every softmax row is
    the same, Delta = n a, W = v for every anchor and H = v: Y = bv Wo + bo everywhere."""
    B, n, h, m, d = 2, 9, 2, 4, 8
    X, _, bqv, U, Wo, bo = _rand(4, B, n, h, m, d)
    C = h * d
    got = oracle.anchor_block_forward(X, np.zeros((C, 2 * C)), bqv, U, Wo, bo)
    want = bqv[C:] @ Wo + bo
    assert np.abs(got - want).max() <= 1e-12 * max(1.0, np.abs(want).max())


def test_head_order_does_not_matter():
    """Relabel the heads (column blocks of Q and V, U's heads, row blocks of Wo): Y is
    unchanged, so no step mixes heads before the output projection."""
    B, n, h, m, d = 2, 11, 3, 4, 8
    X, Wqv, bqv, U, Wo, bo = _rand(5, B, n, h, m, d)
    C = h * d
    perm = [2, 0, 1]
    cols = np.concatenate([np.arange(p * d, (p + 1) * d) for p in perm])
    Wqv2 = np.concatenate([Wqv[:, :C][:, cols], Wqv[:, C:][:, cols]], axis=1)
    bqv2 = np.concatenate([bqv[:C][cols], bqv[C:][cols]])
    got = oracle.anchor_block_forward(X, Wqv2, bqv2, U[perm], Wo[cols, :], bo)
    ref = oracle.anchor_block_forward(X, Wqv, bqv, U, Wo, bo)
    assert _rel(got, ref) <= 1e-13
