"""Pins for the oracle's gradients (dL/dQ, dL/dU, dL/dV for a given dL/dH), each
independent of the oracle's own chain rule.

The gradients are fixed to: central finite differences of the (already pinned) forward,
automatic differentiation of a separately written torch forward in fp64, closed forms
(one anchor: dQ = dU = 0 and dV = token mean of dL/dH; dV = S_t dL/dH with S_t from the
explicit two-step chain), and invariants (shifting every anchor by one vector leaves H
unchanged, so dU sums to zero over the anchors; rows and, by symmetry, columns of S_t sum
to one, so dV and dL/dH have equal column sums).  A dropped term, a wrong sign, a
transposed operand or a missing batch sum for U fails at least one of them.

Sources: AnchorFormer abstract (anchors are learnable, i.e. trained through this layer);
Pith verdict on arXiv 2505.16463 -- referee summary (Eq. 11 / Eq. 12), desk-editor letter
(A row-stochastic, Delta = column sums, S_t 1 = 1), key_machinery (S_t from F^2).
"""
import math

import numpy as np
import pytest

import oracle


def _rel(a, b):
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


def _case(seed, n, m, d, scale=1.0):
    r = np.random.default_rng(seed)
    return (scale * r.standard_normal((n, d)), r.standard_normal((m, d)),
            r.standard_normal((n, d)), r.standard_normal((n, d)))


@pytest.mark.parametrize("seed,n,m,d", [(0, 7, 3, 4), (1, 5, 6, 3), (2, 9, 1, 2), (3, 4, 4, 8)])
def test_gradients_match_finite_differences(seed, n, m, d):
    q, u, v, g = _case(seed, n, m, d, scale=1.5)
    dq, du, dv = oracle.anchor_backward_slice(q, u, v, g)

    def loss(q_, u_, v_):
        return float((oracle.anchor_slice(q_, u_, v_)[3] * g).sum())

    eps = 1e-6
    for name, X, dX in (("q", q, dq), ("u", u, du), ("v", v, dv)):
        num = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            xs = {"q_": q, "u_": u, "v_": v}
            Xp = X.copy(); Xp[idx] += eps
            Xm = X.copy(); Xm[idx] -= eps
            xs[name + "_"] = Xp; lp = loss(**xs)
            xs[name + "_"] = Xm; lm = loss(**xs)
            num[idx] = (lp - lm) / (2 * eps)
        scale = max(np.abs(dX).max(), 1e-3)
        assert np.abs(num - dX).max() / scale <= 1e-6, name


def test_gradients_match_torch_autograd_batched():
    """A separately written fp64 torch forward, differentiated by autograd; U is shared
    by the batch, so its gradient is summed over the batch."""
    torch = pytest.importorskip("torch")
    r = np.random.default_rng(11)
    B, h, n, m, d = 3, 2, 13, 5, 8
    Q, V, G = (r.standard_normal((B, h, n, d)) for _ in range(3))
    U = r.standard_normal((h, m, d))
    tq, tu, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (Q, U, V))
    A = torch.softmax(torch.einsum("bhnd,hmd->bhnm", tq, tu) / math.sqrt(d), dim=-1)
    delta = A.sum(dim=2)                                   # [B, h, m]
    W = torch.einsum("bhnm,bhnd->bhmd", A, tv) / delta[..., None]
    H = torch.einsum("bhnm,bhmd->bhnd", A, W)
    (H * torch.tensor(G)).sum().backward()
    dQ, dU, dV = oracle.anchor_backward(Q, U, V, G)
    assert _rel(dQ, tq.grad.numpy()) <= 1e-11
    assert _rel(dU, tu.grad.numpy()) <= 1e-11
    assert _rel(dV, tv.grad.numpy()) <= 1e-11


def test_single_anchor_closed_form():
    """m = 1: A is all ones, H = token mean of V in every row, so dQ = dU = 0 and every
    row of dV is the token mean of dL/dH."""
    q, u, v, g = _case(4, 11, 1, 6)
    dq, du, dv = oracle.anchor_backward_slice(q, u, v, g)
    assert np.abs(dq).max() <= 1e-14 and np.abs(du).max() <= 1e-14
    assert _rel(dv, np.tile(g.mean(axis=0), (11, 1))) <= 1e-14


@pytest.mark.parametrize("seed", range(5))
def test_value_gradient_is_transition_times_output_gradient(seed):
    """H = S_t V with S_t from the explicit two-step chain (symmetric), so dV = S_t g."""
    q, u, v, g = _case(20 + seed, 12, 4, 5)
    S, _ = oracle.anchor_bruteforce(q, u, v)
    _, _, dv = oracle.anchor_backward_slice(q, u, v, g)
    assert _rel(dv, S @ g) <= 1e-12


@pytest.mark.parametrize("seed", range(5))
def test_invariants(seed):
    q, u, v, g = _case(40 + seed, 16, 6, 7, scale=2.0)
    _, du, dv = oracle.anchor_backward_slice(q, u, v, g)
    # anchor shift invariance: sum over anchors of dU is zero
    assert np.abs(du.sum(axis=0)).max() <= 1e-12 * max(np.abs(du).max(), 1.0)
    # rows and columns of S_t sum to one: dV and g have the same column sums
    assert np.abs(dv.sum(axis=0) - g.sum(axis=0)).max() <= 1e-12 * np.abs(g).sum()


def test_dead_anchor_gradients():
    """An anchor whose softmax column underflows (Delta = 0) gets a zero gradient, and
    the other gradients equal those with the anchor deleted."""
    r = np.random.default_rng(21)
    n, m, d = 30, 5, 16
    q = r.standard_normal((n, d)); q[:, 0] = 5.0 + np.abs(q[:, 0])
    u = r.standard_normal((m, d)); u[2] = 0.0; u[2, 0] = -2000.0 * math.sqrt(d)
    v, g = r.standard_normal((n, d)), r.standard_normal((n, d))
    dq, du, dv = oracle.anchor_backward_slice(q, u, v, g)
    assert np.all(np.isfinite(dq)) and np.all(np.isfinite(du)) and np.all(np.isfinite(dv))
    assert np.all(du[2] == 0.0)
    keep = [i for i in range(m) if i != 2]
    dqk, duk, dvk = oracle.anchor_backward_slice(q, u[keep], v, g)
    assert _rel(dq, dqk) <= 1e-13 and _rel(dv, dvk) <= 1e-13 and _rel(du[keep], duk) <= 1e-13


def test_batched_backward_sums_anchor_gradients_over_the_batch():
    r = np.random.default_rng(5)
    B, h, n, m, d = 4, 3, 9, 3, 4
    Q, V, G = (r.standard_normal((B, h, n, d)) for _ in range(3))
    U = r.standard_normal((h, m, d))
    dQ, dU, dV = oracle.anchor_backward(Q, U, V, G, nthreads=3)
    for hh in range(h):
        acc = np.zeros((m, d))
        for b in range(B):
            dq, du, dv = oracle.anchor_backward_slice(Q[b, hh], U[hh], V[b, hh], G[b, hh])
            assert np.abs(dq - dQ[b, hh]).max() == 0.0 and np.abs(dv - dV[b, hh]).max() == 0.0
            acc += du
        assert np.abs(acc - dU[hh]).max() == 0.0
