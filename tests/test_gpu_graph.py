"""The entry points under HIP graph capture: each call is captured once (after an eager
call of the same shape has sized the workspaces and picked the block's GEMM algorithms),
the graph is replayed several times with eager work and synchronizations between the
replays, and every replay must reproduce the eager result bit for bit.  No entry point
records a memset or an allocation in the graph."""
import numpy as np
import pytest

from efficient_vision_transformer_amd.inputs import make_block_inputs, make_inputs, make_upstream_grad

pytestmark = pytest.mark.gpu


def _conv(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda:0")


def _capture_and_replay(fn, outs, reps=3):
    """fn() enqueues the call writing into the tensors `outs`; returns nothing."""
    import torch
    fn()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    for o in outs:
        o.zero_()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(reps):
        for o in outs:
            o.fill_(float("nan"))
        scratch = torch.randn(1 << 20, device="cuda:0").sum()   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(scratch).item()
        for o, e in zip(outs, eager):
            assert torch.equal(o.view(torch.int16), e.view(torch.int16)), f"replay {rep}"


@pytest.fixture(scope="module")
def ctxs():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from efficient_vision_transformer_amd import AnchorAttention
    out = {p: AnchorAttention(torch.device("cuda:0"), plan=p) for p in ("auto", "split", "fused")}
    yield out
    for c in out.values():
        c.close()


@pytest.mark.parametrize("plan", ["fused", "split"])
def test_forward_graph(ctxs, plan):
    import torch
    x = make_inputs("vit_s16_224", shape={"B": 8})
    Q, U, V = _conv(x.bits["Q"]), _conv(x.bits["U"]), _conv(x.bits["V"])
    H = torch.empty_like(Q)
    print(f"  forward graph plan={plan}", flush=True)
    _capture_and_replay(lambda: ctxs[plan].forward(Q, U, V, out=H), [H])


def test_forward_fp32_long_graph(ctxs):
    import torch
    x = make_inputs("long_16k_fp32", shape={"B": 1, "h": 2, "n": 3000})
    Q, U, V = (torch.from_numpy(a).to("cuda:0") for a in (x.Q, x.U, x.V))
    H = torch.empty_like(Q)
    print("  forward fp32 graph", flush=True)
    _capture_and_replay(lambda: ctxs["auto"].forward(Q, U, V, out=H), [H])


@pytest.mark.parametrize("plan", ["fused", "split"])
def test_backward_graph(ctxs, plan):
    import torch
    x = make_inputs("vit_s16_224", shape={"B": 8})
    _, gb = make_upstream_grad(x, 3)
    Q, U, V, G = _conv(x.bits["Q"]), _conv(x.bits["U"]), _conv(x.bits["V"]), _conv(gb)
    outs = [torch.empty_like(Q), torch.empty_like(U), torch.empty_like(V)]
    print(f"  backward graph plan={plan}", flush=True)
    _capture_and_replay(lambda: ctxs[plan].backward(Q, U, V, G, out=tuple(outs)), outs)


@pytest.mark.parametrize("plan", ["fused", "split"])
def test_linear_graph(ctxs, plan):
    import torch
    x = make_inputs("vit_s16_224", shape={"B": 4})
    Q, K, V = _conv(x.bits["Q"]), _conv(x.bits["K"]), _conv(x.bits["V"])
    O = torch.empty_like(Q)
    print(f"  linear graph plan={plan}", flush=True)
    _capture_and_replay(lambda: ctxs[plan].relu_linear(Q, K, V, out=O), [O])


def test_block_graph(ctxs):
    import torch
    b = make_block_inputs(4, 196, 6, 30, 64, seed=77)
    t = {k: _conv(v) for k, v in b.bits.items()}
    Y = torch.empty_like(t["X"])
    print("  block graph", flush=True)
    _capture_and_replay(lambda: ctxs["auto"].block_forward(t["X"], t["Wqv"], t["bqv"], t["U"],
                                                           t["Wo"], t["bo"], out=Y), [Y])


@pytest.mark.parametrize("s", [32, 64])
def test_nystrom_graph(ctxs, s):
    """Nystrom attention (landmark maxima, landmark pass, solve, output pass) captured."""
    import torch
    from efficient_vision_transformer_amd.inputs import make_landmarks
    x = make_inputs("vit_s16_224", shape={"B": 8, "n": 500})
    Q, K, V = _conv(x.bits["Q"]), _conv(x.bits["K"]), _conv(x.bits["V"])
    idx = torch.from_numpy(make_landmarks(8, 500, s, seed=3)).to("cuda:0")
    H = torch.empty_like(Q)
    print(f"  nystrom graph s={s}", flush=True)
    _capture_and_replay(lambda: ctxs["auto"].nystrom(Q, K, V, idx, out=H), [H])


def test_forward_d128_graph(ctxs):
    """Head dim 128 (split plan) captured."""
    import torch
    from efficient_vision_transformer_amd.inputs import random_case
    x = random_case(5, 2, 2, 700, 64, 128, dtype="bf16")
    Q, U, V = _conv(x.bits["Q"]), _conv(x.bits["U"]), _conv(x.bits["V"])
    H = torch.empty_like(Q)
    print("  forward d=128 graph", flush=True)
    _capture_and_replay(lambda: ctxs["auto"].forward(Q, U, V, out=H), [H])


def test_forward_many_anchors_graph(ctxs):
    """480 anchors (pass 1 and pass 2 on eight waves) captured."""
    import torch
    from efficient_vision_transformer_amd.inputs import random_case
    x = random_case(6, 2, 2, 900, 480, 64, dtype="bf16")
    Q, U, V = _conv(x.bits["Q"]), _conv(x.bits["U"]), _conv(x.bits["V"])
    H = torch.empty_like(Q)
    print("  forward m=480 graph", flush=True)
    _capture_and_replay(lambda: ctxs["auto"].forward(Q, U, V, out=H), [H])
