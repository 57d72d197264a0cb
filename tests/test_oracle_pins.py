"""Pins for the fp64 oracle, independent of the oracle's own formula.

Each test fixes the oracle to something other than itself: the explicit two-step
Markov chain through the anchors, a library softmax, a hand-derived worked example
in exact rational arithmetic, closed forms (mean pooling, cluster means) and the
invariants the AnchorFormer pages state or imply (rows of the two-step transition
sum to one, rank at most m).  Together they are chosen so that a dropped term, a
wrong sign, a wrong normalisation axis or a transposed operand fails at least one.

Sources: Pith verdict on AnchorFormer (arXiv 2505.16463) -- referee summary
(Eq. 11, Eq. 12 order), desk-editor letter (A row-stochastic, Delta = column sums,
S_t 1 = 1), key_machinery (F = D^-1 G, S_t from F^2), pith_inferences (rank <= m),
skeptic critique (Delta^-1 A^T back-transition); AnchorFormer abstract (O(mn)).
"""
from fractions import Fraction
import math

import numpy as np
import pytest
import scipy.special

import oracle


def _rand(seed, n, m, d, scale=1.0):
    rng = np.random.default_rng(seed)
    return (scale * rng.standard_normal((n, d)), rng.standard_normal((m, d)),
            rng.standard_normal((n, d)))


def _rel(a, b):
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


# --- Eq. (12) order equals the explicit two-step chain (Eq. 9 / Eq. 11) --------------

@pytest.mark.parametrize("seed", range(100))
def test_fast_order_equals_bipartite_chain(seed):
    """H = A(Delta^-1(A^T V)) equals (token block of F^2) V with F = D^-1 G."""
    rng = np.random.default_rng(10_000 + seed)
    n = int(rng.integers(1, 97))
    m = int(rng.integers(1, 17))
    d = int(rng.choice([8, 32]))
    scale = float(rng.choice([0.5, 1.0, 3.0]))
    q, u, v = _rand(seed, n, m, d, scale)
    _, _, _, H = oracle.anchor_slice(q, u, v)
    S, Hb = oracle.anchor_bruteforce(q, u, v)
    assert _rel(H, Hb) <= 1e-12
    # Eq. (8) entry formula with the column-normalised back-transition:
    # S_ij = sum_l A_il A_jl / Delta_l, written with a library softmax for A.
    A = scipy.special.softmax(q @ u.T / math.sqrt(d), axis=1)
    S_entry = (A / A.sum(axis=0)) @ A.T
    assert np.abs(S - S_entry).max() <= 1e-12


def test_tiny_workload_chain():
    """The tiny fp32 workload shape (n=64, m=8, d=32) against the explicit chain."""
    from efficient_vision_transformer_amd.inputs import make_inputs
    x = make_inputs("tiny_fp32")
    q, u, v = x.Q[0, 0], x.U[0], x.V[0, 0]
    H = oracle.anchor_attn(x.Q, x.U, x.V)[0, 0]
    _, Hb = oracle.anchor_bruteforce(q, u, v)
    assert _rel(H, Hb) <= 1e-12


# --- a1/a2: the token-anchor attention matrix --------------------------------------

@pytest.mark.parametrize("n,m,d", [(1, 1, 8), (7, 3, 8), (50, 16, 32), (33, 40, 32)])
def test_attention_matrix_is_library_softmax(n, m, d):
    """A = rowsoftmax(Q U^T / sqrt(d)) over anchors, rows sum to one."""
    q, u, v = _rand(n * 31 + m, n, m, d, 2.0)
    A, delta, _, _ = oracle.anchor_slice(q, u, v)
    ref = scipy.special.softmax(q @ u.T / np.sqrt(d), axis=1)
    assert np.abs(A - ref).max() <= 1e-15
    assert np.abs(A.sum(axis=1) - 1).max() <= 1e-14
    assert np.abs(delta - ref.sum(axis=0)).max() <= 1e-13


def test_hand_worked_example():
    """A 2-token, 2-anchor case derived by hand in exact rationals.

    d = 4, anchors u1 = (2,0,0,0), u2 = 0.  Token 1 has q1 = (ln 3, 0, 0, 0), so its
    logits are (ln 3, 0) and its row of A is (3/4, 1/4); token 2 has q2 = 0, row
    (1/2, 1/2).  Delta = (5/4, 3/4).  With V = [[1, 2, 0, -1], [3, -2, 4, 0]]:
    W_1 = (3/4 v1 + 1/2 v2) / (5/4), W_2 = (1/4 v1 + 1/2 v2) / (3/4),
    H_i = A_i1 W_1 + A_i2 W_2."""
    q = np.array([[math.log(3.0), 0, 0, 0], [0, 0, 0, 0]], dtype=np.float64)
    u = np.array([[2.0, 0, 0, 0], [0, 0, 0, 0]])
    V = [[1, 2, 0, -1], [3, -2, 4, 0]]
    F = Fraction
    A = [[F(3, 4), F(1, 4)], [F(1, 2), F(1, 2)]]
    delta = [A[0][0] + A[1][0], A[0][1] + A[1][1]]
    W = [[(A[0][l] * V[0][k] + A[1][l] * V[1][k]) / delta[l] for k in range(4)] for l in range(2)]
    H = [[A[i][0] * W[0][k] + A[i][1] * W[1][k] for k in range(4)] for i in range(2)]
    A_o, delta_o, W_o, H_o = oracle.anchor_slice(q, u, np.array(V, dtype=np.float64))
    assert np.allclose(A_o, np.array(A, dtype=float), rtol=0, atol=1e-15)
    assert np.allclose(delta_o, np.array(delta, dtype=float), rtol=0, atol=1e-15)
    assert np.allclose(W_o, np.array(W, dtype=float), rtol=0, atol=1e-14)
    assert np.allclose(H_o, np.array(H, dtype=float), rtol=0, atol=1e-14)
    # spot value: H_11 = 3/4 * (3/4 + 3/2)/(5/4) + 1/4 * (1/4 + 3/2)/(3/4) = 17/10 + 7/12
    assert H[0][0] == F(3, 4) * F(9, 5) + F(1, 4) * F(7, 3)


# --- structure of the two-step transition S_t = A Delta^-1 A^T -------------------------

@pytest.mark.parametrize("seed", range(5))
def test_transition_structure(seed):
    """Rows of S_t sum to one; S_t is symmetric PSD of rank m; sum of Delta is n."""
    n, m, d = 40, 6, 8
    q, u, v = _rand(seed, n, m, d)
    A, delta, _, _ = oracle.anchor_slice(q, u, v)
    S, _ = oracle.anchor_bruteforce(q, u, v)
    assert np.abs(S.sum(axis=1) - 1).max() <= 1e-14
    assert np.abs(S - S.T).max() <= 1e-15
    ev = np.linalg.eigvalsh(S)
    assert ev.min() >= -1e-13
    assert np.linalg.matrix_rank(S, tol=1e-10) == m
    assert abs(delta.sum() - n) <= 1e-12


def test_rank_bounded_by_tokens_when_anchors_exceed_tokens():
    q, u, v = _rand(3, 5, 9, 8)
    S, _ = oracle.anchor_bruteforce(q, u, v)
    assert np.linalg.matrix_rank(S, tol=1e-10) <= 5
    assert np.abs(S.sum(axis=1) - 1).max() <= 1e-14


@pytest.mark.parametrize("seed", range(3))
def test_constant_values_are_preserved(seed):
    """V = 1 c^T gives H = 1 c^T (row-stochastic transition)."""
    n, m, d = 77, 13, 32
    q, u, _ = _rand(seed, n, m, d, 3.0)
    c = np.random.default_rng(seed).standard_normal(d)
    v = np.tile(c, (n, 1))
    _, _, _, H = oracle.anchor_slice(q, u, v)
    assert np.abs(H - c).max() <= 1e-13


# --- closed forms ------------------------------------------------------------------

def test_mean_pooling_cases():
    """Q = 0, identical anchors, or a single anchor make A uniform: H = mean of V."""
    n, m, d = 31, 7, 16
    q, u, v = _rand(5, n, m, d)
    mean = v.mean(axis=0)
    _, _, _, H = oracle.anchor_slice(np.zeros_like(q), u, v)
    assert np.abs(H - mean).max() <= 1e-14
    _, _, _, H = oracle.anchor_slice(q, np.tile(u[:1], (m, 1)), v)
    assert np.abs(H - mean).max() <= 1e-14
    _, _, _, H = oracle.anchor_slice(q, u[:1], v)
    assert np.abs(H - mean).max() <= 1e-14


def test_one_hot_assignment_gives_cluster_means():
    """Tokens that are large multiples of orthonormal anchors attend to one anchor
    each, so H_i is the mean of V over the tokens assigned to the same anchor."""
    rng = np.random.default_rng(7)
    n, m, d = 60, 5, 32
    basis, _ = np.linalg.qr(rng.standard_normal((d, m)))
    u = basis.T                               # m orthonormal anchors
    assign = rng.integers(0, m, n)
    assign[:m] = np.arange(m)                 # every anchor used
    q = 400.0 * u[assign]
    v = rng.standard_normal((n, d))
    _, _, _, H = oracle.anchor_slice(q, u, v)
    for c in range(m):
        sel = assign == c
        assert np.abs(H[sel] - v[sel].mean(axis=0)).max() <= 1e-12


# --- invariances and linearity -------------------------------------------------------

def test_symmetries_and_linearity():
    n, m, d = 45, 9, 8
    q, u, v = _rand(11, n, m, d, 2.0)
    rng = np.random.default_rng(12)
    _, _, _, H = oracle.anchor_slice(q, u, v)
    # shifting every anchor by one vector adds a per-token constant to the logits
    _, _, _, Hs = oracle.anchor_slice(q, u + rng.standard_normal(d), v)
    assert _rel(Hs, H) <= 1e-12
    # token permutation permutes the output rows
    p = rng.permutation(n)
    _, _, _, Hp = oracle.anchor_slice(q[p], u, v[p])
    assert _rel(Hp, H[p]) <= 1e-13
    # anchor permutation leaves the output unchanged
    _, _, _, Ha = oracle.anchor_slice(q, u[rng.permutation(m)], v)
    assert _rel(Ha, H) <= 1e-13
    # linear in V
    v2 = rng.standard_normal((n, d))
    _, _, _, H2 = oracle.anchor_slice(q, u, v2)
    _, _, _, Hl = oracle.anchor_slice(q, u, 2.5 * v - 0.5 * v2)
    assert _rel(Hl, 2.5 * H - 0.5 * H2) <= 1e-13


def test_dead_anchor_is_removable():
    """An anchor pointing far away from every token gets Delta = 0 (its softmax
    column underflows); its W row is zero and deleting it changes nothing."""
    rng = np.random.default_rng(21)
    n, m, d = 50, 6, 16
    q = rng.standard_normal((n, d))
    q[:, 0] = 5.0 + np.abs(q[:, 0])
    u = rng.standard_normal((m, d))
    u[2] = 0.0
    u[2, 0] = -2000.0 * math.sqrt(d)
    v = rng.standard_normal((n, d))
    A, delta, W, H = oracle.anchor_slice(q, u, v)
    assert delta[2] == 0.0 and np.all(W[2] == 0.0)
    assert np.all(np.isfinite(H))
    keep = [i for i in range(m) if i != 2]
    _, _, _, Hk = oracle.anchor_slice(q, u[keep], v)
    assert np.abs(H - Hk).max() == 0.0
    _, Hb = oracle.anchor_bruteforce(q, u, v)
    assert _rel(H, Hb) <= 1e-12


def test_batched_equals_per_slice():
    """Slices (batch, head) are independent; U is per head, shared over the batch."""
    rng = np.random.default_rng(3)
    B, h, n, m, d = 3, 2, 19, 4, 8
    Q = rng.standard_normal((B, h, n, d))
    V = rng.standard_normal((B, h, n, d))
    U = rng.standard_normal((h, m, d))
    H = oracle.anchor_attn(Q, U, V, nthreads=4)
    for b in range(B):
        for hh in range(h):
            _, _, _, Hs = oracle.anchor_slice(Q[b, hh], U[hh], V[b, hh])
            assert np.abs(H[b, hh] - Hs).max() == 0.0


def test_full_attention_is_textbook():
    """Report-only diagnostic: softmax(QK^T/sqrt(d))V against a library softmax."""
    rng = np.random.default_rng(4)
    n, d = 37, 8
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    ref = scipy.special.softmax(q @ k.T / np.sqrt(d), axis=1) @ v
    full = oracle.full_attention_slice(q, k, v)
    assert np.abs(full - ref).max() <= 1e-13
    rows = [0, 5, 36]
    assert np.abs(oracle.full_attention_slice(q, k, v, rows) - ref[rows]).max() <= 1e-13


def test_errors_are_reported():
    with pytest.raises(RuntimeError):
        oracle.anchor_slice(np.zeros((3, 4)), np.zeros((0, 4)), np.zeros((3, 4)))
    A, delta, W, H = oracle.anchor_slice(np.zeros((0, 4)), np.ones((2, 4)), np.zeros((0, 4)))
    assert H.shape == (0, 4)


def test_golden_tiny_fixture_unchanged():
    """The frozen oracle outputs on the tiny workload (tests/golden) still hold."""
    import os
    from efficient_vision_transformer_amd.inputs import make_inputs
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_fp32_oracle.txt")
    rows = {}
    for line in open(path):
        if line.startswith("#"):
            continue
        key, *vals = line.split()
        rows[key] = np.array([float(v) for v in vals])
    x = make_inputs("tiny_fp32")
    _, delta, _, H = oracle.anchor_slice(x.Q[0, 0], x.U[0], x.V[0, 0])
    assert np.abs(delta - rows["delta"]).max() <= 1e-13
    for r in (0, 17, 63):
        assert np.abs(H[r] - rows[f"H{r}"]).max() <= 1e-13
    assert abs(H.sum() - rows["Hsum"][0]) <= 1e-10
