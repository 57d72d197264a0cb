"""Seeded sweep of random forward shapes over the whole domain, in every plan that accepts
them, against the fp64 oracle: head dims 32/64/128, 1 to 512 anchors, ragged token counts,
fp32 and bf16, Q scaled so that some rows are peaked.  Shapes the plan does not take must
be refused with NOT_SUPPORTED (never a wrong result).  Gates: fp32 normwise max-relative
error <= 1e-5, bf16 relative Frobenius error <= 1e-2."""
import numpy as np
import pytest

import oracle
from efficient_vision_transformer_amd.inputs import random_case

from gpu_util import err_for, tol_for, to_device, to_host

pytestmark = pytest.mark.gpu


def _domain_ok(m, d, dtype):
    """What anchor_attn_forward accepts (its header's domain)."""
    if d == 128 and dtype != "bf16":
        return False
    if m > 256 and (dtype != "bf16" or d > 64):
        return False
    return m <= 512


def _shapes(count, seed):
    r = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        d = int(r.choice([32, 64, 128]))
        dtype = str(r.choice(["fp32", "bf16"]))
        m = int(r.choice([int(r.integers(1, 65)), int(r.integers(65, 257)), int(r.integers(257, 513))]))
        n = int(r.choice([int(r.integers(1, 300)), int(r.integers(300, 2500))]))
        B, h = int(r.integers(1, 4)), int(r.integers(1, 4))
        if _domain_ok(m, d, dtype) and B * h * n * (m + d) <= 6_000_000:
            out.append((B, h, n, m, d, dtype))
    return out


SHAPES = _shapes(40, 20261202)


@pytest.fixture(scope="module")
def ctxs():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from efficient_vision_transformer_amd import AnchorAttention
    dev = torch.device("cuda:0")
    out = {p: AnchorAttention(dev, plan=p) for p in ("auto", "split", "fused")}
    yield dev, out
    for c in out.values():
        c.close()


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_sweep_against_oracle(ctxs, shape):
    import torch
    dev, cs = ctxs
    B, h, n, m, d, dtype = shape
    x = random_case(5000 + SHAPES.index(shape), B, h, n, m, d, dtype=dtype, q_scale=1.5)
    ref = oracle.anchor_attn(x.Q, x.U, x.V)
    Q, U, V = to_device(x, dev)
    for plan in ("auto", "split", "fused"):
        try:
            desc = cs[plan].describe(B, h, n, m, d, dtype)
        except RuntimeError as e:
            assert plan == "fused" and "NOT_SUPPORTED" in str(e), str(e)
            print(f"  {shape} {plan}: refused", flush=True)
            continue
        print(f"  {shape} {plan}: {desc[:60]}", flush=True)
        H = cs[plan].forward(Q, U, V)
        torch.cuda.synchronize()
        e = err_for(dtype, to_host(H), ref)
        print(f"    error {e:.3e}", flush=True)
        assert e <= tol_for(dtype)
