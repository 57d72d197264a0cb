"""Seeded sweep of random backward shapes over the backward's domain (bf16, d = 32 or 64,
1 to 128 anchors, ragged token counts, Q scaled so that some rows are peaked) in every plan
that takes them, against the fp64 oracle's gradients.  Shapes a plan does not take must be
refused with NOT_SUPPORTED.  Gate: relative Frobenius error <= 1e-2 for each of dQ, dU,
dV."""
import numpy as np
import pytest

import oracle
from efficient_vision_transformer_amd.inputs import make_upstream_grad, random_case

from gpu_util import bf16_err, to_device, to_host

pytestmark = pytest.mark.gpu

BWD_TOL = 1e-2


def _shapes(count, seed):
    r = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        d = int(r.choice([32, 64]))
        m = int(r.choice([int(r.integers(1, 65)), int(r.integers(65, 129))]))
        n = int(r.choice([int(r.integers(1, 400)), int(r.integers(400, 2500))]))
        B, h = int(r.integers(1, 4)), int(r.integers(1, 4))
        if B * h * n * (m + d) <= 4_000_000:
            out.append((B, h, n, m, d))
    return out


SHAPES = _shapes(24, 20261203)


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


def _to_dev(bits, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_backward_sweep_against_oracle(ctxs, shape):
    import torch
    dev, cs = ctxs
    B, h, n, m, d = shape
    k = SHAPES.index(shape)
    x = random_case(6000 + k, B, h, n, m, d, "bf16", q_scale=1.5)
    G, gbits = make_upstream_grad(x, 6500 + k)
    ref = oracle.anchor_backward(x.Q, x.U, x.V, G)
    Q, U, V = to_device(x, dev)
    dH = _to_dev(gbits, dev)
    for plan in ("auto", "split", "fused"):
        try:
            dQ, dU, dV = cs[plan].backward(Q, U, V, dH)
        except RuntimeError as e:
            assert plan == "fused" and "NOT_SUPPORTED" in str(e), str(e)
            print(f"  {shape} {plan}: refused", flush=True)
            continue
        torch.cuda.synchronize()
        errs = [bf16_err(to_host(gv), rv) for gv, rv in zip((dQ, dU, dV), ref)]
        print(f"  {shape} {plan}: dQ {errs[0]:.3e} dU {errs[1]:.3e} dV {errs[2]:.3e}", flush=True)
        for name, e in zip(("dQ", "dU", "dV"), errs):
            assert e <= BWD_TOL, f"{shape} {plan} {name}: {e:.3e}"
