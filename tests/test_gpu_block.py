"""GPU parity of the attention block (projections through hipBLASLt around the anchor
attention kernels reading the projection in place) against the oracle's fp64 block on
the same bf16-rounded inputs.  Gate: relative Frobenius error <= 1e-2 (the bf16 gate;
the block rounds the projection and H to bf16 between its steps)."""
import numpy as np
import pytest

import oracle
from efficient_vision_transformer_amd.inputs import make_block_inputs

from gpu_util import bf16_err

pytestmark = pytest.mark.gpu

BLOCK_TOL = 1e-2


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def ctxs(dev):
    from efficient_vision_transformer_amd import AnchorAttention
    out = {p: AnchorAttention(dev, plan=p) for p in ("auto", "split")}
    yield out
    for c in out.values():
        c.close()


def _conv(bits, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def _block(ctx, dev, x, bias=True):
    import torch
    print(f"  block B={x.B} n={x.n} h={x.h} m={x.m} d={x.d} bias={bias} plan={ctx.plan}",
          flush=True)
    t = {k: _conv(v, dev) for k, v in x.bits.items()}
    Y = ctx.block_forward(t["X"], t["Wqv"], t["bqv"] if bias else None, t["U"], t["Wo"],
                          t["bo"] if bias else None)
    torch.cuda.synchronize()
    ref = oracle.anchor_block_forward(x.X, x.Wqv, x.bqv if bias else None, x.U, x.Wo,
                                      x.bo if bias else None)
    e = bf16_err(Y.float().cpu().numpy().astype(np.float64), ref)
    print(f"  relative Frobenius error {e:.3e}", flush=True)
    return e


# (B, n, h, m, d): ViT-S/16 and ViT-B/16 block shapes, ragged token counts, d = 32
SHAPES = [(64, 196, 6, 30, 64), (8, 576, 12, 64, 64), (3, 77, 4, 16, 32), (2, 1000, 2, 100, 64),
          (1, 1, 1, 1, 32)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_block_against_oracle(ctxs, dev, shape):
    B, n, h, m, d = shape
    x = make_block_inputs(B, n, h, m, d, seed=5000 + n + m)
    assert _block(ctxs["auto"], dev, x) <= BLOCK_TOL


def test_block_without_bias_and_split_plan(ctxs, dev):
    x = make_block_inputs(4, 196, 6, 30, 64, seed=5100)
    assert _block(ctxs["auto"], dev, x, bias=False) <= BLOCK_TOL
    assert _block(ctxs["split"], dev, x, bias=True) <= BLOCK_TOL


def test_block_rejects_bad_arguments(ctxs, dev):
    import torch
    ctx = ctxs["auto"]
    x = make_block_inputs(1, 8, 2, 4, 32, seed=5200)
    t = {k: _conv(v, dev) for k, v in x.bits.items()}
    with pytest.raises(RuntimeError, match="status 2"):   # fp32 is not supported
        ctx.block_forward(t["X"].float(), t["Wqv"].float(), None, t["U"].float(),
                          t["Wo"].float(), None)
    with pytest.raises(RuntimeError, match="status 1"):   # output overlapping the input
        ctx.block_forward(t["X"], t["Wqv"], None, t["U"], t["Wo"], None, out=t["X"])
    Y = ctx.block_forward(t["X"], t["Wqv"], t["bqv"], t["U"], t["Wo"], t["bo"])
    torch.cuda.synchronize()
    assert torch.isfinite(Y.float()).all().item()
