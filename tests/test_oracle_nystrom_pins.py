"""Pins of the oracle's Nystrom attention (Fast Nystrom Attention page, key machinery:
three row softmaxes through s landmark rows, the middle one inverted), CPU only.

The oracle evaluates F1 (F2^-1 (F3 V)).  The pins check it against an explicit n x n
chain written in loops with a hand-written Gauss-Jordan inverse, against full softmax
attention when every token is a landmark (the Nystrom product is then exact), and
against closed forms and invariances, so that a transposed factor, a softmax over the
wrong axis, a dropped inverse or a wrong scale each fail one of them."""
import math

import numpy as np
import pytest

import oracle


def _rand(seed, B, h, n, d, scale=1.0):
    r = np.random.default_rng(seed)
    return tuple(scale * r.standard_normal((B, h, n, d)) for _ in range(3))


def _landmarks(seed, B, n, s):
    """Token 0 plus s - 1 distinct other tokens per batch element."""
    r = np.random.default_rng(seed)
    return np.stack([np.concatenate([[0], r.choice(np.arange(1, n), s - 1, replace=False)])
                     for _ in range(B)])


def _softmax_rows_loops(x):
    out = []
    for row in x:
        mx = max(row)
        e = [math.exp(v - mx) for v in row]
        z = sum(e)
        out.append([v / z for v in e])
    return out


def _inverse_gauss_jordan(a):
    n = len(a)
    m = [list(row) + [1.0 if i == j else 0.0 for j in range(n)] for i, row in enumerate(a)]
    for col in range(n):
        piv = max(range(col, n), key=lambda r: abs(m[r][col]))
        m[col], m[piv] = m[piv], m[col]
        p = m[col][col]
        m[col] = [v / p for v in m[col]]
        for r in range(n):
            if r != col:
                f = m[r][col]
                m[r] = [vr - f * vc for vr, vc in zip(m[r], m[col])]
    return [row[n:] for row in m]


@pytest.mark.parametrize("seed,n,s,d", [(0, 9, 3, 4), (1, 12, 5, 3), (2, 7, 7, 2), (3, 10, 1, 5)])
def test_matches_the_explicit_n_by_n_chain_in_loops(seed, n, s, d):
    """H = (F1 F2^-1 F3) V with every factor, the inverse and the n x n product in loops."""
    Q, K, V = _rand(seed, 1, 1, n, d)
    idx = _landmarks(seed + 50, 1, n, s)
    q, k, v, ib = Q[0, 0], K[0, 0], V[0, 0], list(idx[0])
    c = 1.0 / math.sqrt(d)
    dot = lambda a, b: sum(x * y for x, y in zip(a, b))
    F1 = _softmax_rows_loops([[dot(q[i], k[l]) * c for l in ib] for i in range(n)])
    F2 = _softmax_rows_loops([[dot(q[a], k[l]) * c for l in ib] for a in ib])
    F3 = _softmax_rows_loops([[dot(q[a], k[t]) * c for t in range(n)] for a in ib])
    F2i = _inverse_gauss_jordan(F2)
    M = [[sum(F1[i][a] * F2i[a][b] * F3[b][t] for a in range(s) for b in range(s))
          for t in range(n)] for i in range(n)]
    want = np.array([[sum(M[i][t] * v[t][e] for t in range(n)) for e in range(d)]
                     for i in range(n)])
    got = oracle.nystrom_attn(Q, K, V, idx)[0, 0]
    assert np.abs(got - want).max() <= 1e-10 * max(1.0, np.abs(want).max())


@pytest.mark.parametrize("seed,n,d", [(4, 16, 8), (5, 33, 16)])
def test_every_token_a_landmark_gives_full_attention(seed, n, d):
    """With s = n the Nystrom product is F F^-1 F = F, the full attention matrix."""
    Q, K, V = _rand(seed, 1, 2, n, d)
    for idx in (np.arange(n)[None, :], np.random.default_rng(seed).permutation(n)[None, :]):
        got = oracle.nystrom_attn(Q, K, V, idx)
        for j in range(2):
            want = oracle.full_attention_slice(Q[0, j], K[0, j], V[0, j])
            assert np.abs(got[0, j] - want).max() <= 1e-9 * np.abs(want).max()


def test_one_landmark_gives_that_landmark_attention_everywhere():
    """s = 1: F1 and F2 are all ones, so every row is the landmark query's attention
    over all tokens."""
    n, d = 20, 6
    Q, K, V = _rand(6, 1, 1, n, d)
    a = 7
    got = oracle.nystrom_attn(Q, K, V, np.array([[a]]))[0, 0]
    want = oracle.full_attention_slice(Q[0, 0], K[0, 0], V[0, 0], rows=[a])[0]
    assert np.abs(got - want[None, :]).max() <= 1e-12


def test_constant_values_are_preserved():
    """Every factor is row-stochastic and F2^-1 1 = 1, so the rows of F1 F2^-1 F3 sum to
    one: constant V rows give that constant."""
    B, h, n, d, s = 2, 2, 40, 8, 6
    Q, K, _ = _rand(7, B, h, n, d)
    V = np.broadcast_to(np.linspace(-2.0, 3.0, d), (B, h, n, d)).copy()
    got = oracle.nystrom_attn(Q, K, V, _landmarks(7, B, n, s))
    assert np.abs(got - V).max() <= 1e-10


def test_landmark_order_does_not_matter():
    B, h, n, d, s = 2, 2, 30, 8, 5
    Q, K, V = _rand(8, B, h, n, d)
    idx = _landmarks(8, B, n, s)
    perm = np.random.default_rng(9).permutation(s)
    a = oracle.nystrom_attn(Q, K, V, idx)
    b = oracle.nystrom_attn(Q, K, V, idx[:, perm])
    assert np.abs(a - b).max() <= 1e-11 * np.abs(a).max()


def test_token_permutation_permutes_the_output():
    B, h, n, d, s = 1, 2, 25, 8, 4
    Q, K, V = _rand(10, B, h, n, d)
    idx = _landmarks(10, B, n, s)
    perm = np.random.default_rng(11).permutation(n)
    inv = np.argsort(perm)
    a = oracle.nystrom_attn(Q, K, V, idx)
    b = oracle.nystrom_attn(Q[:, :, perm], K[:, :, perm], V[:, :, perm], inv[idx])
    assert np.abs(a[:, :, perm] - b).max() <= 1e-11 * np.abs(a).max()


def test_linear_in_values_and_slices_independent():
    B, h, n, d, s = 2, 3, 18, 4, 3
    Q, K, V = _rand(12, B, h, n, d)
    V2 = _rand(13, B, h, n, d)[2]
    idx = _landmarks(12, B, n, s)
    lhs = oracle.nystrom_attn(Q, K, 2.0 * V - 0.5 * V2, idx)
    rhs = 2.0 * oracle.nystrom_attn(Q, K, V, idx) - 0.5 * oracle.nystrom_attn(Q, K, V2, idx)
    assert np.abs(lhs - rhs).max() <= 1e-10 * np.abs(lhs).max()
    one = oracle.nystrom_attn(Q[1:2, 2:3], K[1:2, 2:3], V[1:2, 2:3], idx[1:2])
    assert np.abs(one[0, 0] - oracle.nystrom_attn(Q, K, V, idx)[1, 2]).max() <= 1e-12


def test_logit_scale_is_one_over_sqrt_d():
    """With s = n the result is softmax(Q K^T / sqrt(d)) V; written out here with d = 9
    (scale 1/3) and Q doubled, so a missing or wrong logit scale fails."""
    n, d = 12, 9
    Q, K, V = _rand(14, 1, 1, n, d)
    got = oracle.nystrom_attn(2.0 * Q, K, V, np.arange(n)[None, :])[0, 0]
    L = (2.0 * Q[0, 0]) @ K[0, 0].T / 3.0
    P = np.exp(L - L.max(axis=1, keepdims=True))
    want = (P / P.sum(axis=1, keepdims=True)) @ V[0, 0]
    assert np.abs(got - want).max() <= 1e-9 * np.abs(want).max()
