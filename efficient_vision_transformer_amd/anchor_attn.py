"""Python binding of the anchor-attention C ABI (include/anchor_attn.h).

Argument marshalling only: torch tensors supply device memory and the current HIP
stream; every step of the computation runs in the HIP kernels of
``libanchor_attn.so``.  There is no CPU fallback -- if the library is missing or
cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
# ANCHOR_ATTN_LIBRARY names another build of the library (the host sanitizer test's)
_LIB_PATH = os.environ.get("ANCHOR_ATTN_LIBRARY") or os.path.join(_HERE, "libanchor_attn.so")

FP32, BF16 = 0, 1
PLAN_AUTO, PLAN_FUSED, PLAN_SPLIT = 0, 1, 2
_PLANS = {"auto": PLAN_AUTO, "fused": PLAN_FUSED, "split": PLAN_SPLIT}

_lib = None
_lib_lock = threading.Lock()


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Loads libanchor_attn.so (once).  Raises RuntimeError if it is not built."""
    global _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"anchor attention HIP library not found at {_LIB_PATH}; build it with "
                "`python -c 'import __graft_entry__ as g; g.build()'`")
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i32 = ctypes.c_void_p, ctypes.c_int
        lib.anchor_attn_create.argtypes = [ctypes.POINTER(vp)]
        lib.anchor_attn_destroy.argtypes = [vp]
        lib.anchor_attn_forward.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]
        lib.anchor_attn_forward_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                                    i32, i32, vp]
        llp = ctypes.POINTER(ctypes.c_longlong)
        lib.anchor_attn_forward_strided.argtypes = [vp, vp, llp, vp, vp, llp, vp, llp,
                                                    i32, i32, i32, i32, i32, i32, vp]
        lib.anchor_attn_relu_linear_forward.argtypes = [vp, vp, llp, vp, llp, vp, llp, vp, llp,
                                                        i32, i32, i32, i32, ctypes.c_float,
                                                        ctypes.c_float, i32, vp]
        lib.anchor_attn_block_forward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp,
                                                  i32, i32, i32, i32, i32, i32, vp]
        lib.anchor_attn_backward_strided.argtypes = [vp, vp, llp, vp, vp, llp, vp, llp, vp, llp,
                                                     vp, vp, llp, i32, i32, i32, i32, i32, i32,
                                                     vp]
        lib.anchor_attn_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp,
                                             i32, i32, i32, i32, i32, i32, vp]
        lib.anchor_attn_nystrom_forward.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                                    i32, i32, vp]
        lib.anchor_attn_set_plan.argtypes = [vp, i32]
        lib.anchor_attn_describe_plan.argtypes = [vp, i32, i32, i32, i32, i32, i32,
                                                  ctypes.c_char_p, i32]
        lib.anchor_attn_status_string.argtypes = [i32]
        lib.anchor_attn_status_string.restype = ctypes.c_char_p
        for f in (lib.anchor_attn_create, lib.anchor_attn_destroy, lib.anchor_attn_forward,
                  lib.anchor_attn_forward_noalloc,
                  lib.anchor_attn_forward_strided, lib.anchor_attn_block_forward,
                  lib.anchor_attn_relu_linear_forward, lib.anchor_attn_backward_strided,
                  lib.anchor_attn_backward, lib.anchor_attn_nystrom_forward,
                  lib.anchor_attn_set_plan,
                  lib.anchor_attn_describe_plan):
            f.restype = i32
        _lib = lib
        return lib


def status_string(code: int) -> str:
    return load_library().anchor_attn_status_string(int(code)).decode()


def _check(code: int, what: str) -> None:
    if code != 0:
        raise RuntimeError(f"{what}: {status_string(code)} (status {code})")


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return FP32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"anchor attention supports float32 and bfloat16, got {t.dtype}")


class AnchorAttention:
    """Owns one library context (and its workspace) on one device."""

    def __init__(self, device=None, plan: str = "auto"):
        import torch
        self.device = torch.device("cuda", torch.cuda.current_device() if device is None
                                   else torch.device(device).index or 0)
        lib = load_library()
        handle = ctypes.c_void_p()
        with torch.cuda.device(self.device):
            _check(lib.anchor_attn_create(ctypes.byref(handle)), "anchor_attn_create")
        self._h = handle
        self._lib = lib
        self.plan = "auto"
        if plan != "auto":
            self.set_plan(plan)

    def set_plan(self, plan: str) -> None:
        _check(self._lib.anchor_attn_set_plan(self._h, _PLANS[plan]), "anchor_attn_set_plan")
        self.plan = plan

    def describe(self, B, h, n, m, d, dtype: str = "bf16") -> str:
        buf = ctypes.create_string_buffer(512)
        code = FP32 if dtype == "fp32" else BF16
        _check(self._lib.anchor_attn_describe_plan(self._h, B, h, n, m, d, code, buf, 512),
               "anchor_attn_describe_plan")
        return buf.value.decode()

    def forward(self, Q, U, V, out=None, stream=None):
        """Q, V: [B, h, n, d]; U: [h, m, d] contiguous; same dtype, on this device.
        Q, V and ``out`` may be strided views (say the halves of a packed [B, n, 2, h, d]
        projection, or an output view of a [B, n, h, d] tensor) as long as the d values
        of each token are contiguous.  Returns H [B, h, n, d] (``out`` if given, else a
        new contiguous tensor).  Enqueued on ``stream`` (default: the current torch
        stream); no synchronisation."""
        import torch
        if Q.dim() != 4 or V.shape != Q.shape or U.dim() != 3:
            raise ValueError(f"bad shapes Q{tuple(Q.shape)} U{tuple(U.shape)} V{tuple(V.shape)}")
        B, h, n, d = Q.shape
        if U.shape[0] != h or U.shape[2] != d:
            raise ValueError(f"U must be [h={h}, m, d={d}], got {tuple(U.shape)}")
        m = U.shape[1]
        for name, t in (("Q", Q), ("U", U), ("V", V)):
            if not t.is_cuda or t.device != self.device:
                raise ValueError(f"{name} must live on {self.device}")
            if t.dtype != Q.dtype:
                raise TypeError("Q, U and V must share one dtype")
        if not U.is_contiguous():
            raise ValueError("U must be contiguous")
        if out is None:
            out = torch.empty(Q.shape, dtype=Q.dtype, device=Q.device)
        elif out.shape != Q.shape or out.dtype != Q.dtype or out.device != self.device:
            raise ValueError("out must be a tensor of Q's shape, dtype and device")
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        sv = ctypes.c_void_p(stream.cuda_stream)
        if Q.is_contiguous() and V.is_contiguous() and out.is_contiguous():
            _check(self._lib.anchor_attn_forward(
                self._h, Q.data_ptr(), U.data_ptr(), V.data_ptr(), out.data_ptr(),
                B, h, n, m, d, _dtype_code(Q), sv), "anchor_attn_forward")
            return out
        strides = []
        for name, t in (("Q", Q), ("V", V), ("out", out)):
            if t.stride(3) != 1 and d > 1:
                raise ValueError(f"{name}: the d values of a token must be contiguous")
            strides.append((ctypes.c_longlong * 3)(t.stride(0), t.stride(1), t.stride(2)))
        _check(self._lib.anchor_attn_forward_strided(
            self._h, Q.data_ptr(), strides[0], U.data_ptr(), V.data_ptr(), strides[1],
            out.data_ptr(), strides[2], B, h, n, m, d, _dtype_code(Q), sv),
            "anchor_attn_forward_strided")
        return out

    __call__ = forward

    def forward_noalloc(self, Q, U, V, out, stream=None):
        """forward() through anchor_attn_forward_noalloc: the split plan's partials live in
        the library's fixed 64 MiB scratch on this GPU instead of this context's workspace,
        so the call allocates nothing (``out`` must be given).  Contiguous tensors only.
        Calls that may overlap on one GPU share that scratch and race."""
        if Q.dim() != 4 or V.shape != Q.shape or U.dim() != 3 or out.shape != Q.shape:
            raise ValueError(f"bad shapes Q{tuple(Q.shape)} U{tuple(U.shape)} V{tuple(V.shape)}")
        B, h, n, d = Q.shape
        if U.shape[0] != h or U.shape[2] != d:
            raise ValueError(f"U must be [h={h}, m, d={d}], got {tuple(U.shape)}")
        for name, t in (("Q", Q), ("U", U), ("V", V), ("out", out)):
            if not t.is_cuda or t.device != self.device or t.dtype != Q.dtype:
                raise ValueError(f"{name} must be a {Q.dtype} tensor on {self.device}")
            if not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous")
        if stream is None:
            import torch
            stream = torch.cuda.current_stream(self.device)
        _check(self._lib.anchor_attn_forward_noalloc(
            self._h, Q.data_ptr(), U.data_ptr(), V.data_ptr(), out.data_ptr(), B, h, n,
            U.shape[1], d, _dtype_code(Q), ctypes.c_void_p(stream.cuda_stream)),
            "anchor_attn_forward_noalloc")
        return out

    def relu_linear(self, Q, K, V, cmin: float = 100.0, qscale: float = 1.0, out=None,
                    stream=None):
        """ReLU kernel linear attention: relu(qscale q_i) (relu(K)^T V) /
        max(relu(qscale q_i) . relu(K)^T 1, cmin) per (batch, head) slice.  Q, K, V and
        ``out`` are [B, h, n, d] bf16 tensors or views whose d values per token are
        contiguous.  Returns out (a new contiguous tensor unless given)."""
        import torch
        if Q.dim() != 4 or K.shape != Q.shape or V.shape != Q.shape:
            raise ValueError(f"bad shapes Q{tuple(Q.shape)} K{tuple(K.shape)} V{tuple(V.shape)}")
        B, h, n, d = Q.shape
        if out is None:
            out = torch.empty(Q.shape, dtype=Q.dtype, device=Q.device)
        elif out.shape != Q.shape or out.dtype != Q.dtype:
            raise ValueError("out must be a tensor of Q's shape and dtype")
        strides = []
        for name, t in (("Q", Q), ("K", K), ("V", V), ("out", out)):
            if not t.is_cuda or t.device != self.device or t.dtype != Q.dtype:
                raise ValueError(f"{name} must be a {Q.dtype} tensor on {self.device}")
            if t.stride(3) != 1 and d > 1:
                raise ValueError(f"{name}: the d values of a token must be contiguous")
            strides.append((ctypes.c_longlong * 3)(t.stride(0), t.stride(1), t.stride(2)))
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        _check(self._lib.anchor_attn_relu_linear_forward(
            self._h, Q.data_ptr(), strides[0], K.data_ptr(), strides[1], V.data_ptr(),
            strides[2], out.data_ptr(), strides[3], B, h, n, d, float(cmin), float(qscale),
            _dtype_code(Q), ctypes.c_void_p(stream.cuda_stream)),
            "anchor_attn_relu_linear_forward")
        return out

    def nystrom(self, Q, K, V, idx, out=None, stream=None):
        """Nystrom attention with given landmarks: F1 (F2^-1 (F3 V)) per (batch, head)
        slice with F1 = rowsoftmax(Q k^T c), F2 = rowsoftmax(q k^T c), F3 = rowsoftmax(q K^T c),
        q, k the rows idx[b] of Q, K and c = 1/sqrt(d).  Q, K, V contiguous [B, h, n, d] bf16;
        idx an int32 [B, s] tensor of token indices on the same device.  Returns out (a new
        tensor unless given)."""
        import torch
        if Q.dim() != 4 or K.shape != Q.shape or V.shape != Q.shape:
            raise ValueError(f"bad shapes Q{tuple(Q.shape)} K{tuple(K.shape)} V{tuple(V.shape)}")
        B, h, n, d = Q.shape
        if idx.dim() != 2 or idx.shape[0] != B or idx.dtype != torch.int32:
            raise ValueError("idx must be an int32 tensor [B, s]")
        if out is None:
            out = torch.empty(Q.shape, dtype=Q.dtype, device=Q.device)
        elif out.shape != Q.shape or out.dtype != Q.dtype:
            raise ValueError("out must be a tensor of Q's shape and dtype")
        for name, t in (("Q", Q), ("K", K), ("V", V), ("idx", idx), ("out", out)):
            if not t.is_cuda or t.device != self.device:
                raise ValueError(f"{name} must be on {self.device}")
            if not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous")
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        _check(self._lib.anchor_attn_nystrom_forward(
            self._h, Q.data_ptr(), K.data_ptr(), V.data_ptr(), idx.data_ptr(), out.data_ptr(),
            B, h, n, idx.shape[1], d, _dtype_code(Q), ctypes.c_void_p(stream.cuda_stream)),
            "anchor_attn_nystrom_forward")
        return out

    def block_forward(self, X, Wqv, bqv, U, Wo, bo, out=None, stream=None):
        """The attention block: Y = anchor_attention(X Wqv + bqv split into Q | V) Wo + bo.
        X [B, n, C] (C = h*d), Wqv [C, 2C], bqv [2C] or None, U [h, m, d], Wo [C, C],
        bo [C] or None; bf16, contiguous, on this device.  Returns Y [B, n, C] (``out`` if
        given)."""
        import torch
        if X.dim() != 3 or U.dim() != 3:
            raise ValueError(f"bad shapes X{tuple(X.shape)} U{tuple(U.shape)}")
        B, n, C = X.shape
        h, m, d = U.shape
        if h * d != C or Wqv.shape != (C, 2 * C) or Wo.shape != (C, C):
            raise ValueError(f"need C = h*d and Wqv [C, 2C], Wo [C, C]: X{tuple(X.shape)} "
                             f"U{tuple(U.shape)} Wqv{tuple(Wqv.shape)} Wo{tuple(Wo.shape)}")
        if bqv is not None and bqv.shape != (2 * C,):
            raise ValueError("bqv must be [2C]")
        if bo is not None and bo.shape != (C,):
            raise ValueError("bo must be [C]")
        for name, t in (("X", X), ("Wqv", Wqv), ("bqv", bqv), ("U", U), ("Wo", Wo), ("bo", bo)):
            if t is None:
                continue
            if not t.is_cuda or t.device != self.device or not t.is_contiguous() or t.dtype != X.dtype:
                raise ValueError(f"{name} must be a contiguous {X.dtype} tensor on {self.device}")
        if out is None:
            out = torch.empty_like(X)
        elif out.shape != X.shape or out.dtype != X.dtype or not out.is_contiguous() \
                or out.device != self.device:
            raise ValueError("out must be a contiguous tensor like X")
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        ptr = lambda t: None if t is None else t.data_ptr()
        _check(self._lib.anchor_attn_block_forward(
            self._h, X.data_ptr(), Wqv.data_ptr(), ptr(bqv), U.data_ptr(), Wo.data_ptr(),
            ptr(bo), out.data_ptr(), B, n, h, m, d, _dtype_code(X),
            ctypes.c_void_p(stream.cuda_stream)), "anchor_attn_block_forward")
        return out

    def backward(self, Q, U, V, dH, out=None, stream=None):
        """Gradients for dL/dH = dH: returns (dQ [B,h,n,d], dU [h,m,d] summed over the
        batch, dV [B,h,n,d]) in the inputs' dtype (bf16 or fp32), enqueued on ``stream``; no
        synchronisation.  Q, V, dH (and dQ, dV in ``out``) may be strided views whose d
        values per token are contiguous; U and dU are contiguous.  ``out`` may give (dQ, dU, dV) to write into."""
        import torch
        if Q.dim() != 4 or V.shape != Q.shape or dH.shape != Q.shape or U.dim() != 3:
            raise ValueError(f"bad shapes Q{tuple(Q.shape)} U{tuple(U.shape)} V{tuple(V.shape)} "
                             f"dH{tuple(dH.shape)}")
        B, h, n, d = Q.shape
        if U.shape[0] != h or U.shape[2] != d:
            raise ValueError(f"U must be [h={h}, m, d={d}], got {tuple(U.shape)}")
        m = U.shape[1]
        for name, t in (("Q", Q), ("U", U), ("V", V), ("dH", dH)):
            if not t.is_cuda or t.device != self.device:
                raise ValueError(f"{name} must live on {self.device}")
            if t.dtype != Q.dtype:
                raise TypeError("Q, U, V and dH must share one dtype")
        if not U.is_contiguous():
            raise ValueError("U must be contiguous")
        if out is None:
            dQ = torch.empty(Q.shape, dtype=Q.dtype, device=Q.device)
            dU = torch.empty_like(U)
            dV = torch.empty(Q.shape, dtype=Q.dtype, device=Q.device)
        else:
            dQ, dU, dV = out
            for name, t, like in (("dQ", dQ, Q), ("dU", dU, U), ("dV", dV, V)):
                if t.shape != like.shape or t.dtype != like.dtype or t.device != like.device:
                    raise ValueError(f"{name} must be a {like.dtype} tensor of shape "
                                     f"{tuple(like.shape)} on {like.device}")
            if not dU.is_contiguous():
                raise ValueError("dU must be contiguous")
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        sv = ctypes.c_void_p(stream.cuda_stream)
        views = (Q, V, dH, dQ, dV)
        if all(t.is_contiguous() for t in views):
            _check(self._lib.anchor_attn_backward(
                self._h, Q.data_ptr(), U.data_ptr(), V.data_ptr(), dH.data_ptr(), dQ.data_ptr(),
                dU.data_ptr(), dV.data_ptr(), B, h, n, m, d, _dtype_code(Q), sv),
                "anchor_attn_backward")
            return dQ, dU, dV
        st = []
        for name, t in zip(("Q", "V", "dH", "dQ", "dV"), views):
            if t.stride(3) != 1 and d > 1:
                raise ValueError(f"{name}: the d values of a token must be contiguous")
            st.append((ctypes.c_longlong * 3)(t.stride(0), t.stride(1), t.stride(2)))
        _check(self._lib.anchor_attn_backward_strided(
            self._h, Q.data_ptr(), st[0], U.data_ptr(), V.data_ptr(), st[1], dH.data_ptr(), st[2],
            dQ.data_ptr(), st[3], dU.data_ptr(), dV.data_ptr(), st[4], B, h, n, m, d,
            _dtype_code(Q), sv), "anchor_attn_backward_strided")
        return dQ, dU, dV

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            self._lib.anchor_attn_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


_shared: dict = {}
_shared_lock = threading.Lock()


def shared_context(device, stream=None) -> AnchorAttention:
    """The module's context for (device, stream): one per stream, because calls on one
    context that run concurrently on different streams would share its workspace.  The
    stream defaults to torch's current stream on `device`.  A context serves one host thread
    at a time; the lock covers the lookup, callers on several threads and one stream must
    serialise their calls themselves."""
    import torch
    dev = torch.device(device)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    key = (dev.index if dev.index is not None else torch.cuda.current_device(), stream.cuda_stream)
    with _shared_lock:
        ctx = _shared.get(key)
        if ctx is None:
            ctx = _shared[key] = AnchorAttention(dev)
        return ctx


def forward(Q, U, V, out=None, stream=None):
    """H = A (Delta^-1 (A^T V)) with A = rowsoftmax(Q U^T / sqrt(d)), on Q's device and
    `stream` (default: torch's current stream), with that stream's shared context."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(Q.device)
    return shared_context(Q.device, stream).forward(Q, U, V, out=out, stream=stream)
