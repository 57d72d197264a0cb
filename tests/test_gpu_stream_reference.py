"""The measurement helper anchor_attn_stream_reference (include/anchor_attn_bench.h):
c = a ^ b over the given bytes, nothing written past them, argument errors refused."""
import ctypes

import pytest

pytestmark = pytest.mark.gpu


def test_stream_reference_xors_exactly_the_given_bytes():
    import torch
    from efficient_vision_transformer_amd import anchor_attn
    lib = anchor_attn.load_library()
    fn = lib.anchor_attn_stream_reference
    fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_longlong,
                   ctypes.c_void_p]
    fn.restype = ctypes.c_int
    g = torch.Generator(device="cuda:0").manual_seed(3)
    n = 1000 * 8 + 24                      # int16 elements: a ragged last workgroup
    a = torch.randint(-30000, 30000, (n,), dtype=torch.int16, device="cuda:0", generator=g)
    b = torch.randint(-30000, 30000, (n,), dtype=torch.int16, device="cuda:0", generator=g)
    c = torch.full((n + 64,), 7, dtype=torch.int16, device="cuda:0")
    assert fn(a.data_ptr(), b.data_ptr(), c.data_ptr(), 2 * n, None) == 0
    torch.cuda.synchronize()
    assert torch.equal(c[:n], torch.bitwise_xor(a, b))
    assert torch.all(c[n:] == 7)
    assert fn(a.data_ptr(), b.data_ptr(), c.data_ptr(), 2 * n - 2, None) == 1   # not a multiple of 16
    assert fn(a.data_ptr() + 2, b.data_ptr(), c.data_ptr(), 16, None) == 1      # misaligned
    assert fn(a.data_ptr(), b.data_ptr(), c.data_ptr(), 0, None) == 0           # no-op
