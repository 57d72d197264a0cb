"""Pins of the oracle's ReLU linear attention (L2ViT page, Eq. (4) with phi = ReLU and
the Cmin clamp), CPU only.  The oracle evaluates the associative order
phi(Q) (phi(K)^T V); the pins check it against the quadratic order written out in loops,
closed forms and invariances chosen so that a swapped operand, a missing ReLU, a missing
clamp or a wrong normalisation each fail one of them."""
import numpy as np
import pytest

import oracle


def _rand(seed, B, h, n, d, scale=1.0):
    r = np.random.default_rng(seed)
    return tuple(scale * r.standard_normal((B, h, n, d)) for _ in range(3))


@pytest.mark.parametrize("seed,cmin", [(0, 100.0), (1, 1.0), (2, 1e-6), (3, 30.0)])
def test_matches_the_quadratic_order_in_loops(seed, cmin):
    """out_i = sum_j w_ij v_j / max(sum_j w_ij, cmin) with w_ij = relu(q_i) . relu(k_j)."""
    B, h, n, d = 2, 2, 7, 5
    Q, K, V = _rand(seed, B, h, n, d, scale=2.0)
    want = np.zeros_like(Q)
    for b in range(B):
        for j in range(h):
            for i in range(n):
                qi = [max(x, 0.0) for x in Q[b, j, i]]
                wsum, acc = 0.0, [0.0] * d
                for t in range(n):
                    w = sum(qi[e] * max(K[b, j, t, e], 0.0) for e in range(d))
                    wsum += w
                    for e in range(d):
                        acc[e] += w * V[b, j, t, e]
                den = max(wsum, cmin)
                want[b, j, i] = [a / den for a in acc]
    got = oracle.relu_linear_attn(Q, K, V, cmin=cmin)
    assert np.abs(got - want).max() <= 1e-12 * max(1.0, np.abs(want).max())


def test_unclamped_rows_are_convex_combinations():
    """With the clamp inactive the weights of each row sum to one: constant V rows give
    that constant, and every output lies within V's per-dim range."""
    B, h, n, d = 1, 2, 30, 8
    Q, K, _ = _rand(4, B, h, n, d)
    Q = np.abs(Q) + 0.5
    K = np.abs(K) + 0.5                        # all weights positive and large
    V = np.broadcast_to(np.arange(d, dtype=float), (B, h, n, d)).copy()
    out = oracle.relu_linear_attn(Q, K, V, cmin=1e-9)
    assert np.abs(out - V).max() <= 1e-12 * d
    V2 = _rand(5, B, h, n, d)[2]
    out2 = oracle.relu_linear_attn(Q, K, V2, cmin=1e-9)
    assert np.all(out2 <= V2.max(axis=2, keepdims=True) + 1e-12)
    assert np.all(out2 >= V2.min(axis=2, keepdims=True) - 1e-12)


def test_negative_queries_or_keys_give_zero():
    Q, K, V = _rand(6, 1, 1, 9, 4)
    assert np.all(oracle.relu_linear_attn(-np.abs(Q), K, V) == 0.0)
    assert np.all(oracle.relu_linear_attn(Q, -np.abs(K), V) == 0.0)


def test_clamp_binds_for_small_weights():
    """Tiny positive weights: the denominator is cmin, so out = relu(q) S / cmin."""
    B, h, n, d = 1, 1, 6, 3
    Q, K, V = _rand(7, B, h, n, d)
    Q, K = 1e-3 * np.abs(Q), 1e-3 * np.abs(K)
    S = K[0, 0].T @ V[0, 0]
    out = oracle.relu_linear_attn(Q, K, V, cmin=100.0)
    assert np.allclose(out[0, 0], Q[0, 0] @ S / 100.0, rtol=1e-13, atol=0)


def test_query_scale_only_moves_the_clamp():
    Q, K, V = _rand(8, 2, 2, 12, 6)
    a = 0.125
    got = oracle.relu_linear_attn(Q, K, V, cmin=3.0, qscale=a)
    assert np.allclose(got, oracle.relu_linear_attn(Q, K, V, cmin=3.0 / a), rtol=1e-13, atol=1e-15)


def test_token_permutations():
    """Permuting the keys and values together changes nothing; permuting the queries
    permutes the output rows."""
    Q, K, V = _rand(9, 1, 2, 15, 6)
    p = np.random.default_rng(1).permutation(15)
    base = oracle.relu_linear_attn(Q, K, V, cmin=2.0)
    assert np.allclose(oracle.relu_linear_attn(Q, K[:, :, p], V[:, :, p], cmin=2.0), base,
                       rtol=1e-13, atol=1e-15)
    assert np.allclose(oracle.relu_linear_attn(Q[:, :, p], K, V, cmin=2.0), base[:, :, p],
                       rtol=1e-13, atol=1e-15)
