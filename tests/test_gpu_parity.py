"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle, element by
element, on seeded inputs.

Gates: fp32 normwise max-relative error <= 1e-5, bf16 relative Frobenius error <= 1e-2
(inputs rounded once to the storage dtype; the oracle reads the rounded values, so the
comparison measures kernel error only).
"""
import numpy as np
import pytest

import oracle
from efficient_vision_transformer_amd.inputs import WORKLOADS, make_inputs, random_case

from gpu_util import err_for, tol_for, to_device, to_host

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


def _run(ctx, x, dev):
    import torch
    Q, U, V = to_device(x, dev)
    print(f"  forward {x.workload.name} B={x.workload.B} h={x.workload.h} n={x.workload.n} "
          f"m={x.workload.m} d={x.workload.d} {x.workload.dtype}", flush=True)
    H = ctx.forward(Q, U, V)
    torch.cuda.synchronize()
    return to_host(H)


# --- the six workload runs ----------------------------------------------------------------

def test_tiny_fp32_against_chain(ctxs, dev):
    """Tiny fp32 workload against both the fast-order oracle and the explicit F^2 chain."""
    x = make_inputs("tiny_fp32")
    got = _run(ctxs["auto"], x, dev)
    ref = oracle.anchor_attn(x.Q, x.U, x.V)
    _, chain = oracle.anchor_bruteforce(x.Q[0, 0], x.U[0], x.V[0, 0])
    assert err_for("fp32", got, ref) <= 1e-5
    assert err_for("fp32", got[0, 0], chain) <= 1e-5


@pytest.mark.parametrize("name", ["vit_s16_224", "vit_b16_384"])
def test_vit_workloads_full(ctxs, dev, name):
    """ViT-shaped workloads, every output element against the oracle."""
    x = make_inputs(name)
    got = _run(ctxs["auto"], x, dev)
    ref = oracle.anchor_attn(x.Q, x.U, x.V)
    e = err_for("bf16", got, ref)
    print(f"  {name}: rel Frobenius {e:.3e}")
    assert e <= 1e-2
    # worst single slice as well
    per = [err_for("bf16", got[b, j], ref[b, j]) for b in range(x.workload.B) for j in range(x.workload.h)]
    assert max(per) <= 1e-2


@pytest.mark.parametrize("name", ["dense_64x64", "long_16k_bf16", "long_16k_fp32"])
def test_large_workloads_every_slice(ctxs, dev, name):
    """Full-size large workloads in the benchmarked launch configuration; the oracle
    computes every slice (fp64, all host threads), and every slice meets the gate."""
    x = make_inputs(name, with_k=False)
    w = x.workload
    got = _run(ctxs["auto"], x, dev)
    assert np.all(np.isfinite(got))
    ref = oracle.anchor_attn(x.Q, x.U, x.V)
    e = err_for(w.dtype, got, ref)
    print(f"  {name}: whole tensor {e:.3e}", flush=True)
    assert e <= tol_for(w.dtype)
    per = [err_for(w.dtype, got[b, j], ref[b, j]) for b in range(w.B) for j in range(w.h)]
    print(f"  {name}: worst slice {max(per):.3e}", flush=True)
    assert max(per) <= tol_for(w.dtype)


# --- edge shapes and both plans -------------------------------------------------------------

EDGE = [
    # (B, h, n, m, d)
    (1, 1, 1, 1, 32), (1, 1, 15, 7, 64), (1, 1, 17, 30, 32), (1, 7, 196, 33, 64),
    (7, 1, 577, 64, 64), (1, 1, 129, 256, 64), (2, 3, 300, 1, 64), (1, 1, 5, 40, 32),
    (1, 1, 1000, 100, 64), (1, 2, 2051, 128, 32),
    # m > 128 is padded to a multiple of 64: padding spread over the last four tiles
    (1, 2, 300, 130, 64), (2, 1, 257, 200, 32), (1, 1, 77, 193, 64),
    # six anchor tiles: the token-split pass 1 takes its generic per-tile operand reads
    (1, 2, 200, 80, 64), (1, 1, 150, 70, 32),
    # the split plan's chunking at its ends: more slices than CUs (one chunk per slice,
    # twelve rounds in pass 1) and two slices cut into many chunks
    (75, 4, 1500, 100, 64), (1, 2, 12000, 200, 64),
]


def _fused_applies(shape, dtype):
    B, h, n, m, d = shape
    return dtype == "bf16" and m <= 64 and n <= 1024


# Every (plan, shape, dtype) combination the plan accepts; the fused plan's refusal of
# the others is checked by test_fused_plan_rejects_what_it_cannot_run.
EDGE_CASES = [
    pytest.param(plan, shape, dtype, id=f"{plan}-{'x'.join(map(str, shape))}-{dtype}")
    for plan in ("auto", "split", "fused")
    for shape in EDGE
    for dtype in ("fp32", "bf16")
    if plan != "fused" or _fused_applies(shape, dtype)
]


@pytest.mark.parametrize("plan,shape,dtype", EDGE_CASES)
def test_edge_shapes(ctxs, dev, shape, dtype, plan):
    B, h, n, m, d = shape
    x = random_case(7 + n + m, B, h, n, m, d, dtype=dtype, q_scale=1.5)
    got = _run(ctxs[plan], x, dev)
    ref = oracle.anchor_attn(x.Q, x.U, x.V)
    e = err_for(dtype, got, ref)
    assert e <= tol_for(dtype), e


def test_empty_inputs_are_noops(ctxs, dev):
    import torch
    ctx = ctxs["auto"]
    for B, h, n in ((0, 2, 10), (2, 0, 10), (2, 2, 0)):
        Q = torch.zeros((B, h, n, 64), device=dev, dtype=torch.bfloat16)
        U = torch.ones((h, 8, 64), device=dev, dtype=torch.bfloat16)
        H = ctx.forward(Q, U, Q.clone())
        torch.cuda.synchronize()
        assert H.shape == Q.shape


FUSED_EXTRA = [(3, 2, 32, 32, 64), (1, 1, 33, 64, 64), (2, 1, 512, 32, 64), (1, 2, 513, 31, 64),
               (1, 1, 1024, 64, 64), (2, 2, 700, 50, 32), (1, 1, 96, 2, 32)]


@pytest.mark.parametrize("shape", FUSED_EXTRA, ids=lambda s: "x".join(map(str, s)))
def test_fused_plan_shapes(ctxs, dev, shape):
    """Pair counts on both sides of the kept-A / recompute switch, ragged tails."""
    B, h, n, m, d = shape
    x = random_case(100 + n, B, h, n, m, d, dtype="bf16", q_scale=2.0)
    got = _run(ctxs["fused"], x, dev)
    ref = oracle.anchor_attn(x.Q, x.U, x.V)
    assert err_for("bf16", got, ref) <= 1e-2


# Slice counts around the CU count: with d = 64 the fused plan lets two workgroups share
# up to 2 * CUs - slices slices (one per half of the output dims), pairing workgroup ids in
# runs of 16 with a neighbour-pair tail.  These counts cover: all slices shared, complete
# runs plus a tail, a single shared slice, and none shared.
SHARED_SLICES = [(1, 1), (3, 3), (9, 1), (4, 25), (50, 6), (100, 3), (64, 6), (73, 7),
                 (128, 4), (130, 4)]


@pytest.mark.parametrize("m", [30, 64])
@pytest.mark.parametrize("bh", SHARED_SLICES, ids=lambda t: f"{t[0]}x{t[1]}")
def test_fused_shared_slices(ctxs, dev, bh, m):
    B, h = bh
    ctx = ctxs["fused"]
    plan = ctx.describe(B, h, 40, m, 64, "bf16")
    print(f"  {plan}", flush=True)
    x = random_case(500 + B * h + m, B, h, 40, m, 64, dtype="bf16", q_scale=1.5)
    got = _run(ctx, x, dev)
    ref = oracle.anchor_attn(x.Q, x.U, x.V)
    assert err_for("bf16", got, ref) <= 1e-2
    # every slice on its own: a mis-paired half would leave one slice far off
    for b in range(B):
        for hh in range(h):
            assert err_for("bf16", got[b, hh], ref[b, hh]) <= 1e-2, (b, hh)


def test_fused_plan_rejects_what_it_cannot_run(ctxs, dev):
    import torch
    Q = torch.zeros((1, 1, 64, 64), device=dev, dtype=torch.float32)
    U = torch.zeros((1, 8, 64), device=dev, dtype=torch.float32)
    with pytest.raises(RuntimeError, match="NOT_SUPPORTED"):
        ctxs["fused"].forward(Q, U, Q.clone())
    Qb = torch.zeros((1, 1, 64, 64), device=dev, dtype=torch.bfloat16)
    Ub = torch.zeros((1, 100, 64), device=dev, dtype=torch.bfloat16)
    with pytest.raises(RuntimeError, match="NOT_SUPPORTED"):
        ctxs["fused"].forward(Qb, Ub, Qb.clone())


def test_headline_plans_agree(ctxs, dev):
    """Fused and split plans on the ViT-S/16 workload both meet the gate."""
    x = make_inputs("vit_s16_224", with_k=False)
    ref = oracle.anchor_attn(x.Q, x.U, x.V)
    for plan in ("fused", "split"):
        assert err_for("bf16", _run(ctxs[plan], x, dev), ref) <= 1e-2, plan


# --- properties that hold at any size --------------------------------------------------

def test_constant_values_preserved_full_size(ctxs, dev):
    """Rows of A Delta^-1 A^T sum to one, so V = 1 c^T gives H = 1 c^T."""
    import torch
    for name in ("vit_s16_224", "dense_64x64"):
        x = make_inputs(name, with_k=False)
        Q, U, _ = to_device(x, dev)
        c = torch.linspace(-2, 2, x.workload.d, device=dev).to(Q.dtype)
        V = c.expand_as(Q).contiguous()
        H = ctxs["auto"].forward(Q, U, V)
        torch.cuda.synchronize()
        err = (H.float() - c.float()).abs().max().item()
        assert err <= 2.0 * 1e-2, (name, err)


def test_deterministic_bitwise(ctxs, dev):
    """Two runs on the same inputs give bitwise-equal outputs (no float atomics)."""
    import torch
    for name in ("vit_s16_224", "dense_64x64"):
        x = make_inputs(name, with_k=False)
        Q, U, V = to_device(x, dev)
        H1 = ctxs["auto"].forward(Q, U, V).clone()
        H2 = ctxs["auto"].forward(Q, U, V)
        torch.cuda.synchronize()
        assert torch.equal(H1.view(torch.int16), H2.view(torch.int16)), name


def test_nan_stays_in_its_slice(ctxs, dev):
    import torch
    x = random_case(3, 2, 2, 200, 30, 64, dtype="bf16")
    Q, U, V = to_device(x, dev)
    H0 = ctxs["split"].forward(Q, U, V).clone()
    V[1, 0, 5, 3] = float("nan")
    H1 = ctxs["split"].forward(Q, U, V)
    torch.cuda.synchronize()
    assert torch.isnan(H1[1, 0]).any()
    for b, j in ((0, 0), (0, 1), (1, 1)):
        assert torch.equal(H1[b, j].view(torch.int16), H0[b, j].view(torch.int16))


# --- C ABI error paths (nothing is enqueued) ---------------------------------------------

def test_abi_rejects_bad_arguments(ctxs, dev):
    import ctypes
    import torch
    from efficient_vision_transformer_amd import anchor_attn
    lib = anchor_attn.load_library()
    h = ctxs["auto"]._h
    Q = torch.zeros((1, 1, 64, 64), device=dev, dtype=torch.bfloat16)
    V = torch.zeros_like(Q)
    U = torch.zeros((1, 16, 64), device=dev, dtype=torch.bfloat16)
    H = torch.full_like(Q, 7.0)
    p = lambda t, off=0: ctypes.c_void_p(t.data_ptr() + off)
    call = lambda *a: lib.anchor_attn_forward(h, *a, None)
    args = lambda **kw: dict(dict(Q=p(Q), U=p(U), V=p(V), H=p(H), B=1, hh=1, n=64, m=16, d=64, dt=1), **kw)
    def run(**kw):
        a = args(**kw)
        return call(a["Q"], a["U"], a["V"], a["H"], a["B"], a["hh"], a["n"], a["m"], a["d"], a["dt"])
    assert run() == 0
    torch.cuda.synchronize()
    H.fill_(7.0)
    torch.cuda.synchronize()
    assert run(Q=None) == 1
    assert run(m=0) == 1
    assert run(n=-1) == 1
    assert run(d=48) == 2
    assert run(m=513) == 2
    assert run(dt=5) == 2
    assert run(H=p(Q)) == 1            # output aliases an input
    assert run(V=p(V, 2)) == 1         # misaligned
    torch.cuda.synchronize()
    assert torch.all(H == 7.0)         # nothing ran on error
