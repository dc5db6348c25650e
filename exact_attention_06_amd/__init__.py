"""MI355X (gfx950) exact-attention forward pass: Python binding of libfa.so.

    o, lse = forward(q, k, v, causal=False, scale=None)
    dq, dk, dv = backward(q, k, v, o, lse, dout, causal=False, scale=None)

q [B, Nq, Hq, d], k/v [B, Nk, Hkv, d] (bf16 or fp16, contiguous, on the GPU);
returns o [B, Nq, Hq, d] (same dtype) and lse [B, Hq, Nq] (fp32). torch provides device
memory and the current stream; the computation is entirely the library's HIP kernels.
Contract violations raise (ValueError for arguments, RuntimeError for launch failures);
nothing falls back to another implementation.
"""

from __future__ import annotations

import math

from . import _lib

__all__ = ["forward", "backward", "check_args", "FaError"]


class FaError(ValueError):
    def __init__(self, code, msg):
        super().__init__(f"fa_fwd: {msg} (code {code})")
        self.code = code


def _raise(code):
    if code == _lib.FA_ERR_LAUNCH:
        raise RuntimeError(f"fa_fwd: {_lib.strerror(code)} (code {code})")
    raise FaError(code, _lib.strerror(code))


def check_args(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, Nq, Nk, Hq, Hkv, d, causal, scale) -> int:
    """Host-only validation (fa_fwd_check): returns the status fa_fwd would return."""
    return _lib.load().fa_fwd_check(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, Nq, Nk, Hq, Hkv, d,
                                    int(bool(causal)), float(scale))


def forward(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None):
    import torch

    lib = _lib.load()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on the GPU")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [batch, seq, heads, head_dim]")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k and v must share one dtype")
    if q.dtype == torch.bfloat16:
        fn = lib.fa_fwd
    elif q.dtype == torch.float16:
        fn = lib.fa_fwd_f16
    else:
        raise ValueError("dtype must be bfloat16 or float16")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k and v must be on one device")
    B, Nq, Hq, d = q.shape
    Bk, Nk, Hkv, dk = k.shape
    if Bk != B or dk != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError("q/k/v shapes do not match: q [B,Nq,Hq,d], k and v [B,Nk,Hkv,d]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous tensor like q")
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    elif (tuple(lse.shape) != (B, Hq, Nq) or lse.dtype != torch.float32 or not lse.is_contiguous()
          or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 tensor [B, Hq, Nq]")
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        rc = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                B, Nq, Nk, Hq, Hkv, d, int(bool(causal)), float(scale), stream)
    if rc != 0:
        _raise(rc)
    return out, lse


def _check_tensor(name, t, torch):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def backward(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None):
    """Gradients (dq, dk, dv) of sum(o * dout) for o, lse = forward(q, k, v, causal, scale)."""
    import torch

    lib = _lib.load()
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse), ("dout", dout)):
        _check_tensor(name, t, torch)
    if not (q.dtype == k.dtype == v.dtype == o.dtype == dout.dtype):
        raise ValueError("q, k, v, o and dout must share one dtype")
    if q.dtype == torch.bfloat16:
        fn = lib.fa_bwd
    elif q.dtype == torch.float16:
        fn = lib.fa_bwd_f16
    else:
        raise ValueError("dtype must be bfloat16 or float16")
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be 4-D [batch, seq, heads, head_dim]")
    B, Nq, Hq, d = q.shape
    Bk, Nk, Hkv, dk_ = k.shape
    if Bk != B or dk_ != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError("q/k/v shapes do not match: q [B,Nq,Hq,d], k and v [B,Nk,Hkv,d]")
    if tuple(o.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape):
        raise ValueError("o and dout must have the shape of q")
    if tuple(lse.shape) != (B, Hq, Nq) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B, Hq, Nq]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    nbytes = int(lib.fa_bwd_workspace_bytes(B, Nq, Hq))
    ws = torch.empty(max(1, nbytes // 4), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        rc = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), nbytes, B, Nq, Nk, Hq, Hkv, d,
                int(bool(causal)), float(scale), stream)
    if rc != 0:
        _raise(rc)
    return dq, dk, dv
