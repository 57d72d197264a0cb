"""GPU parity on the method's own special cases, through the C ABI, in every plan that
takes them, against the fp64 oracle (whose values these cases pin by closed forms in
test_oracle_pins.py) and against the closed forms themselves:

* a dead anchor (its softmax column underflows to exactly 0, so its column sum Delta is
  0 and it must contribute nothing: reading R8 of the Pith verdict page's Eq. (11)),
  equal to the call with that anchor deleted;
* uniform A (Q = 0, identical anchors, a single anchor): H is the token mean of V, i.e.
  mean pooling, since rows of A Delta^-1 A^T then hold 1/n everywhere;
* one-hot A (tokens that are large multiples of orthonormal anchors): H_i is the mean of
  V over the tokens assigned to the same anchor (cluster means);
* a NaN stays inside its (batch, head) slice in the fused plan too, including slices
  shared by two workgroups (one per half of the output dims) and head dim 128.

Gates: fp32 normwise max-relative error <= 1e-5, bf16 relative Frobenius error <= 1e-2.
"""
import math

import numpy as np
import pytest

import oracle
from efficient_vision_transformer_amd.inputs import bf16_bits_rne, bf16_bits_to_f32

from gpu_util import err_for, tol_for, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def ctxs(dev):
    from efficient_vision_transformer_amd import AnchorAttention
    out = {p: AnchorAttention(dev, plan=p) for p in ("auto", "split", "fused")}
    yield out
    for c in out.values():
        c.close()


def _store(a, dtype):
    """float64 -> (exact stored values as float64, device tensor) in `dtype`."""
    import torch
    a32 = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "fp32":
        return a32.astype(np.float64), torch.from_numpy(a32)
    bits = bf16_bits_rne(a32)
    return (bf16_bits_to_f32(bits).astype(np.float64),
            torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16))


def _run(ctx, dev, Q, U, V, dtype, label):
    """Stores Q, U, V in `dtype`, runs the forward, returns (H, Qs, Us, Vs) where the
    last three are the stored values the oracle must read."""
    import torch
    (Qs, Qt), (Us, Ut), (Vs, Vt) = (_store(a, dtype) for a in (Q, U, V))
    B, h, n, d = Q.shape
    print(f"  {label}: plan={ctx.plan} B={B} h={h} n={n} m={U.shape[1]} d={d} {dtype} "
          f"-> {ctx.describe(B, h, n, U.shape[1], d, dtype).split(';')[0]}", flush=True)
    H = ctx.forward(Qt.to(dev), Ut.to(dev), Vt.to(dev))
    torch.cuda.synchronize()
    return to_host(H), Qs, Us, Vs


# (plan, B, h, n, m, d, dtype): the fused plan (bf16, n <= 1024, m <= 64) at d = 32, 64 and
# 128, with whole and shared slices; the split plan in bf16 (token-split and anchor-split
# pass 1) and fp32.
CASES = [
    ("fused", 2, 3, 196, 30, 64, "bf16"),
    ("fused", 3, 2, 577, 64, 64, "bf16"),
    ("fused", 2, 2, 100, 20, 32, "bf16"),
    ("fused", 1, 3, 250, 30, 128, "bf16"),
    ("split", 2, 3, 196, 30, 64, "bf16"),
    ("split", 1, 2, 1500, 128, 64, "bf16"),
    ("split", 1, 2, 700, 200, 64, "bf16"),
    ("split", 1, 2, 300, 40, 128, "bf16"),
    ("split", 2, 3, 196, 30, 64, "fp32"),
    ("split", 1, 2, 900, 150, 32, "fp32"),
]
IDS = ["-".join(map(str, c)) for c in CASES]


def _gate(dtype, got, ref, what):
    e = err_for(dtype, got, ref)
    print(f"    {what}: {e:.3e}", flush=True)
    assert e <= tol_for(dtype), (what, e)


def _m_pad(m):
    """The kernels' anchor padding: a multiple of 32 up to 128 anchors, of 64 up to 256,
    of 128 beyond."""
    step = 32 if m <= 128 else (64 if m <= 256 else 128)
    return -(-m // step) * step


# --- a dead anchor ----------------------------------------------------------------------

def _dead_anchor_inputs(seed, B, h, n, m, d, dead):
    """Every token has a large positive first coordinate; anchor `dead` points the other
    way along it, 2000 sqrt(d) long, so its logits sit ~1e4 below every row maximum and
    its softmax column is exactly 0 in fp32 and fp64 alike."""
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((B, h, n, d))
    Q[..., 0] = 5.0 + np.abs(Q[..., 0])
    U = rng.standard_normal((h, m, d))
    U[:, dead, :] = 0.0
    U[:, dead, 0] = -2000.0 * math.sqrt(d)
    V = rng.standard_normal((B, h, n, d))
    return Q, U, V


@pytest.mark.parametrize("plan,B,h,n,m,d,dtype", CASES, ids=IDS)
def test_dead_anchor_contributes_nothing(ctxs, dev, plan, B, h, n, m, d, dtype):
    ctx = ctxs[plan]
    for dead in (m // 2, m - 1):
        Q, U, V = _dead_anchor_inputs(31 + n + m + dead, B, h, n, m, d, dead)
        got, Qs, Us, Vs = _run(ctx, dev, Q, U, V, dtype, f"dead anchor {dead}")
        assert np.all(np.isfinite(got))
        ref = oracle.anchor_attn(Qs, Us, Vs)
        _gate(dtype, got, ref, "against the oracle")
        # the anchor deleted: same answer (from the oracle and from the kernels)
        keep = [a for a in range(m) if a != dead]
        ref_del = oracle.anchor_attn(Qs, np.ascontiguousarray(Us[:, keep]), Vs)
        assert np.abs(ref - ref_del).max() == 0.0   # the oracle's own pin, on these inputs
        got_del, *_ = _run(ctx, dev, Q, np.ascontiguousarray(U[:, keep]), V, dtype,
                           "same, anchor deleted")
        _gate(dtype, got, got_del, "against the kernels without the anchor")
        if dead == m - 1 and _m_pad(m) == _m_pad(m - 1):
            # the last anchor: with it deleted it becomes padding of the same tile, and a
            # zero softmax weight adds exactly nothing anywhere
            assert np.array_equal(got, got_del)


# --- uniform A: mean pooling --------------------------------------------------------------

@pytest.mark.parametrize("plan,B,h,n,m,d,dtype", CASES, ids=IDS)
def test_uniform_attention_is_mean_pooling(ctxs, dev, plan, B, h, n, m, d, dtype):
    ctx = ctxs[plan]
    rng = np.random.default_rng(5 + n + m)
    Q = rng.standard_normal((B, h, n, d))
    U = rng.standard_normal((h, m, d))
    V = rng.standard_normal((B, h, n, d))
    variants = {
        "Q = 0": (np.zeros_like(Q), U),
        "identical anchors": (Q, np.repeat(U[:, :1], m, axis=1)),
        "one anchor": (Q, np.ascontiguousarray(U[:, :1])),
    }
    for what, (q, u) in variants.items():
        got, Qs, Us, Vs = _run(ctx, dev, q, u, V, dtype, what)
        mean = np.broadcast_to(Vs.mean(axis=2, keepdims=True), Vs.shape)
        _gate(dtype, got, oracle.anchor_attn(Qs, Us, Vs), f"{what}: against the oracle")
        _gate(dtype, got, mean, f"{what}: against the token mean of V")


# --- one-hot A: cluster means -------------------------------------------------------------

# m orthonormal anchors need m <= d
ONE_HOT = [c for c in CASES if c[4] <= c[5]]


@pytest.mark.parametrize("plan,B,h,n,m,d,dtype", ONE_HOT, ids=["-".join(map(str, c)) for c in ONE_HOT])
def test_one_hot_attention_gives_cluster_means(ctxs, dev, plan, B, h, n, m, d, dtype):
    ctx = ctxs[plan]
    rng = np.random.default_rng(7 + n + m)
    U = np.empty((h, m, d))
    for j in range(h):
        basis, _ = np.linalg.qr(rng.standard_normal((d, m)))
        U[j] = basis.T
    assign = rng.integers(0, m, (B, h, n))
    assign[..., :m] = np.arange(m)            # every anchor used in every slice
    Q = 400.0 * np.stack([np.stack([U[j][assign[b, j]] for j in range(h)]) for b in range(B)])
    V = rng.standard_normal((B, h, n, d))
    got, Qs, Us, Vs = _run(ctx, dev, Q, U, V, dtype, "one-hot")
    means = np.empty_like(Vs)
    for b in range(B):
        for j in range(h):
            for a in range(m):
                sel = assign[b, j] == a
                means[b, j, sel] = Vs[b, j, sel].mean(axis=0)
    _gate(dtype, got, oracle.anchor_attn(Qs, Us, Vs), "against the oracle")
    _gate(dtype, got, means, "against the cluster means")


# --- NaN isolation in the fused plan --------------------------------------------------------

@pytest.mark.parametrize("d", [64, 128])
def test_fused_nan_stays_in_its_slice(ctxs, dev, d):
    """ViT-S/16 slice count (384 on 256 CUs: 128 slices shared by two workgroups at d = 64,
    every slice at d = 128).  A NaN in V reaches only its own slice (and, for a shared
    slice, only the half of the dims that reads it); a NaN in Q reaches its whole slice."""
    import torch
    from efficient_vision_transformer_amd.inputs import random_case
    from gpu_util import to_device
    ctx = ctxs["fused"]
    B, h, n, m = 64, 6, 196, 30
    plan = ctx.describe(B, h, n, m, d, "bf16")
    print(f"  {plan}", flush=True)
    assert plan.startswith("fused")
    x = random_case(91 + d, B, h, n, m, d, dtype="bf16")
    Q, U, V = to_device(x, dev)
    H0 = ctx.forward(Q, U, V).clone()
    torch.cuda.synchronize()
    same = lambda a, b: torch.equal(a.view(torch.int16), b.view(torch.int16))
    # last slice (shared at both head dims), a whole slice at d = 64 (slice 3)
    for b, j in ((B - 1, h - 1), (0, 3)):
        for where in ("V", "Q"):
            Qn, Vn = Q.clone(), V.clone()
            tgt = Vn if where == "V" else Qn
            tgt[b, j, 17, 5] = float("nan")
            H1 = ctx.forward(Qn, U, Vn)
            torch.cuda.synchronize()
            nan = torch.isnan(H1.float())
            assert nan[b, j].any(), (where, b, j)
            if where == "Q":
                # the NaN token's row of A is NaN, and so is its row of H
                assert nan[b, j, 17].all(), (b, j)
            else:
                # only column 5 of A^T V is NaN: H's dim 5 in every token, nothing else
                assert nan[b, j, :, 5].all() and nan[b, j].sum().item() == n, (b, j)
            mask = torch.ones((B, h), dtype=torch.bool)
            mask[b, j] = False
            assert same(H1[mask], H0[mask]), (where, b, j)
