"""Helpers for the GPU tests: moving seeded inputs to the device and the error metrics.

Error metrics (tolerances from the anchor-attention parity gates):
  fp32: normwise max-relative error  max|H - H_ref| / max|H_ref|  <= 1e-5
  bf16: relative Frobenius error     ||H - H_ref||_F / ||H_ref||_F  <= 1e-2
Elementwise relative error is not used: entries of H cancel towards 0.
"""
import numpy as np

FP32_TOL = 1e-5
BF16_TOL = 1e-2


def to_device(x, dev):
    """Inputs -> (Q, U, V) device tensors in the workload's storage dtype."""
    import torch
    if x.workload.dtype == "bf16":
        conv = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(dev)
        return conv(x.bits["Q"]), conv(x.bits["U"]), conv(x.bits["V"])
    return tuple(torch.from_numpy(np.ascontiguousarray(a)).to(dev) for a in (x.Q, x.U, x.V))


def to_host(H):
    return H.float().cpu().numpy().astype(np.float64)


def fp32_err(got, ref):
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-300))


def bf16_err(got, ref):
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def err_for(dtype, got, ref):
    return fp32_err(got, ref) if dtype == "fp32" else bf16_err(got, ref)


def tol_for(dtype):
    return FP32_TOL if dtype == "fp32" else BF16_TOL
