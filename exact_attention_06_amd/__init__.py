"""MI355X (gfx950) exact-attention forward pass: Python binding of libfa.so.

    o, lse = forward(q, k, v, causal=False, scale=None)
    dq, dk, dv = backward(q, k, v, o, lse, dout, causal=False, scale=None)
    o, lse = forward_splitkv(q, k, v, causal=False, scale=None, num_splits=None)
    o, lse = forward_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, causal=False,
                            scale=None, seqused_k=None)
    o, lse = forward_paged(q, k_cache, v_cache, cu_seqlens_q, seqused_k, block_table,
                           max_seqlen_q, causal=False, scale=None)

q [B, Nq, Hq, d], k/v [B, Nk, Hkv, d] (bf16 or fp16, contiguous, on the GPU);
returns o [B, Nq, Hq, d] (same dtype) and lse [B, Hq, Nq] (fp32). The variable-length
forms take packed q [total_q, Hq, d] and return o like q and lse [Hq, total_q]; their causal
mask is aligned bottom-right (see include/fa_fwd.h). torch provides device
memory and the current stream; the computation is entirely the library's HIP kernels.
Contract violations raise (ValueError for arguments, RuntimeError for launch failures);
nothing falls back to another implementation.
"""

from __future__ import annotations

import math

from . import _lib

__all__ = ["forward", "set_grid_order", "forward_fp8", "forward_splitkv", "num_splits", "backward", "forward_varlen",
           "forward_paged", "var_num_splits", "check_args", "FaError"]


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


def forward_fp8(q, k, v, q_scale: float = 1.0, k_scale: float = 1.0, v_scale: float = 1.0,
                causal: bool = False, scale: float | None = None):
    """Forward pass on e4m3 inputs (fa_fwd_fp8): q [B, Nq, Hq, d], k/v [B, Nk, Hkv, d] as
    torch.float8_e4m3fn with one dequantisation factor each; returns o [B, Nq, Hq, d] in
    bfloat16 and lse [B, Hq, Nq] (fp32) of attention on q_scale*q, k_scale*k, v_scale*v."""
    import torch

    lib = _lib.load()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, torch)
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [batch, seq, heads, head_dim]")
        if t.dtype != torch.float8_e4m3fn:
            raise ValueError(f"{name} must be torch.float8_e4m3fn")
        if t.device != q.device:
            raise ValueError("q, k and v must be on one device")
    B, Nq, Hq, d = q.shape
    Bk, Nk, Hkv, dk = k.shape
    if Bk != B or dk != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError("q/k/v shapes do not match: q [B,Nq,Hq,d], k and v [B,Nk,Hkv,d]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty((B, Nq, Hq, d), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        rc = lib.fa_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                            float(q_scale), float(k_scale), float(v_scale), B, Nq, Nk, Hq, Hkv, d,
                            int(bool(causal)), float(scale), stream)
    if rc != 0:
        _raise(rc)
    return out, lse


def set_grid_order(mul: int = 0, add: int = 0) -> None:
    """Grid order of every later launch in this process (testing hook for races between
    workgroups): workgroup i takes work item (i * m + add) mod n, m the first value >= mul mod n
    coprime with the grid size n; (0, 0) is the natural order."""
    rc = _lib.load().fa_set_grid_order(int(mul) & 0xFFFFFFFF, int(add) & 0xFFFFFFFF)
    if rc:
        _raise(rc)


def num_splits(B, Nq, Nk, Hq, d, causal=False) -> int:
    """The library's split count for a shape (fa_fwd_num_splits; 1 = no split)."""
    return int(_lib.load().fa_fwd_num_splits(B, Nq, Nk, Hq, d, int(bool(causal))))


def forward_splitkv(q, k, v, causal: bool = False, scale: float | None = None, num_splits=None):
    """forward() with the key range of every query tile split over num_splits workgroups
    (fa_fwd_splitkv); num_splits=None takes the library's choice. The workspace is
    allocated here with torch."""
    import torch

    lib = _lib.load()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, torch)
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [batch, seq, heads, head_dim]")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k and v must share one dtype")
    if q.dtype == torch.bfloat16:
        fn = lib.fa_fwd_splitkv
    elif q.dtype == torch.float16:
        fn = lib.fa_fwd_splitkv_f16
    else:
        raise ValueError("dtype must be bfloat16 or float16")
    B, Nq, Hq, d = q.shape
    Bk, Nk, Hkv, dk = k.shape
    if Bk != B or dk != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError("q/k/v shapes do not match: q [B,Nq,Hq,d], k and v [B,Nk,Hkv,d]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if num_splits is None:
        num_splits = int(lib.fa_fwd_num_splits(B, Nq, Nk, Hq, d, int(bool(causal))))
    nbytes = int(lib.fa_fwd_splitkv_workspace_bytes(B, Nq, Hq, d, int(num_splits)))
    ws = torch.empty(max(4, nbytes // 4), dtype=torch.float32, device=q.device)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        rc = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), ws.data_ptr(), nbytes,
                B, Nq, Nk, Hq, Hkv, d, int(bool(causal)), float(scale), int(num_splits), stream)
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


def backward(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None, noalloc: bool = False):
    """Gradients (dq, dk, dv) of sum(o * dout) for o, lse = forward(q, k, v, causal, scale).

    noalloc=True calls fa_bwd_noalloc (bf16 only): no workspace, D kept in the library's
    fixed device scratch (calls that overlap on one GPU race on it)."""
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
    if noalloc:
        if q.dtype != torch.bfloat16:
            raise ValueError("the allocation-free backward pass takes bfloat16 tensors")
        with torch.cuda.device(q.device):
            stream = torch.cuda.current_stream(q.device).cuda_stream
            rc = lib.fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                    dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Nq, Nk, Hq, Hkv,
                                    d, int(bool(causal)), float(scale), stream)
        if rc != 0:
            _raise(rc)
        return dq, dk, dv
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


def _int32_vec(name, t, n, torch, device):
    _check_tensor(name, t, torch)
    if t.dtype != torch.int32 or t.dim() != 1 or t.shape[0] != n:
        raise ValueError(f"{name} must be a 1-D int32 tensor with {n} entries")
    if t.device != device:
        raise ValueError(f"{name} must be on the device of q")


def _varlen_common(q, kv_tensors, torch, lib, bf16_fn, f16_fn):
    for name, t in (("q", q),) + kv_tensors:
        _check_tensor(name, t, torch)
        if t.device != q.device:
            raise ValueError("all tensors must be on one device")
    if any(t.dtype != q.dtype for _, t in kv_tensors):
        raise ValueError("q, k and v must share one dtype")
    if q.dtype == torch.bfloat16:
        return getattr(lib, bf16_fn)
    if q.dtype == torch.float16:
        return getattr(lib, f16_fn)
    raise ValueError("dtype must be bfloat16 or float16")


def _varlen_out(q, out, lse, torch):
    total_q, Hq, _ = q.shape
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous tensor like q")
    if lse is None:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    elif (tuple(lse.shape) != (Hq, total_q) or lse.dtype != torch.float32 or not lse.is_contiguous()
          or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 tensor [Hq, total_q]")
    return out, lse


def var_num_splits(B: int, max_seqlen_q: int, key_bound: int, Hq: int, d: int) -> int:
    """The library's split count for a variable-length / paged batch (fa_fwd_var_num_splits);
    key_bound bounds every sequence's key count (paged: max_pages * page_size). 0: no split."""
    return int(_lib.load().fa_fwd_var_num_splits(B, max_seqlen_q, key_bound, Hq, d))


def _var_workspace(lib, total_q, Hq, d, num_splits, q, torch):
    nbytes = lib.fa_fwd_var_splitkv_workspace_bytes(total_q, Hq, d, int(num_splits))
    if nbytes == 0:
        raise ValueError("num_splits must be a positive integer")
    return torch.empty(nbytes // 4, dtype=torch.float32, device=q.device), nbytes


def forward_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, causal: bool = False,
                   scale: float | None = None, seqused_k=None, out=None, lse=None, num_splits: int = 0):
    """Packed variable-length forward (fa_fwd_varlen): q [total_q, Hq, d], k/v [total_k, Hkv, d],
    cu_seqlens_q / cu_seqlens_k int32 [B+1], seqused_k None or int32 [B]. Returns
    o [total_q, Hq, d] and lse [Hq, total_q] (fp32). num_splits > 0 cuts every sequence's keys
    into chunks over that many split-KV blocks (fa_fwd_varlen_splitkv; workspace allocated here)."""
    import torch

    lib = _lib.load()
    if num_splits:
        fn = _varlen_common(q, (("k", k), ("v", v)), torch, lib, "fa_fwd_varlen_splitkv",
                            "fa_fwd_varlen_splitkv_f16")
    else:
        fn = _varlen_common(q, (("k", k), ("v", v)), torch, lib, "fa_fwd_varlen", "fa_fwd_varlen_f16")
    if q.dim() != 3 or k.dim() != 3 or tuple(v.shape) != tuple(k.shape) or k.shape[2] != q.shape[2]:
        raise ValueError("q must be [total_q, Hq, d] and k, v [total_k, Hkv, d]")
    total_q, Hq, d = q.shape
    total_k, Hkv, _ = k.shape
    B = cu_seqlens_q.shape[0] - 1 if isinstance(cu_seqlens_q, torch.Tensor) else -1
    _int32_vec("cu_seqlens_q", cu_seqlens_q, B + 1, torch, q.device)
    _int32_vec("cu_seqlens_k", cu_seqlens_k, B + 1, torch, q.device)
    if seqused_k is not None:
        _int32_vec("seqused_k", seqused_k, B, torch, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, lse = _varlen_out(q, out, lse, torch)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        used = 0 if seqused_k is None else seqused_k.data_ptr()
        if num_splits:
            ws, nbytes = _var_workspace(lib, total_q, Hq, d, num_splits, q, torch)
            rc = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), ws.data_ptr(), nbytes,
                    cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), used, B, int(max_seqlen_q), total_q, total_k,
                    Hq, Hkv, d, int(bool(causal)), float(scale), int(num_splits), stream)
        else:
            rc = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                    cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), used, B, int(max_seqlen_q), total_q, total_k,
                    Hq, Hkv, d, int(bool(causal)), float(scale), stream)
    if rc != 0:
        _raise(rc)
    return out, lse


def forward_paged(q, k_cache, v_cache, cu_seqlens_q, seqused_k, block_table, max_seqlen_q: int,
                  causal: bool = False, scale: float | None = None, out=None, lse=None, num_splits: int = 0):
    """Forward against a paged K/V cache (fa_fwd_paged): q [total_q, Hq, d],
    k_cache/v_cache [num_pages, page_size, Hkv, d], cu_seqlens_q int32 [B+1], seqused_k
    int32 [B], block_table int32 [B, max_pages]. Returns o [total_q, Hq, d] and
    lse [Hq, total_q] (fp32). num_splits > 0 cuts every sequence's keys into chunks over that
    many split-KV blocks (fa_fwd_paged_splitkv; workspace allocated here)."""
    import torch

    lib = _lib.load()
    if num_splits:
        fn = _varlen_common(q, (("k_cache", k_cache), ("v_cache", v_cache)), torch, lib, "fa_fwd_paged_splitkv",
                            "fa_fwd_paged_splitkv_f16")
    else:
        fn = _varlen_common(q, (("k_cache", k_cache), ("v_cache", v_cache)), torch, lib, "fa_fwd_paged",
                            "fa_fwd_paged_f16")
    if (q.dim() != 3 or k_cache.dim() != 4 or tuple(v_cache.shape) != tuple(k_cache.shape)
            or k_cache.shape[3] != q.shape[2]):
        raise ValueError("q must be [total_q, Hq, d] and k_cache, v_cache [num_pages, page_size, Hkv, d]")
    total_q, Hq, d = q.shape
    num_pages, page_size, Hkv, _ = k_cache.shape
    B = cu_seqlens_q.shape[0] - 1 if isinstance(cu_seqlens_q, torch.Tensor) else -1
    _int32_vec("cu_seqlens_q", cu_seqlens_q, B + 1, torch, q.device)
    _int32_vec("seqused_k", seqused_k, B, torch, q.device)
    _check_tensor("block_table", block_table, torch)
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be an int32 tensor [B, max_pages]")
    if block_table.device != q.device:
        raise ValueError("block_table must be on the device of q")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, lse = _varlen_out(q, out, lse, torch)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        if num_splits:
            ws, nbytes = _var_workspace(lib, total_q, Hq, d, num_splits, q, torch)
            rc = fn(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(), lse.data_ptr(),
                    ws.data_ptr(), nbytes, cu_seqlens_q.data_ptr(), seqused_k.data_ptr(), block_table.data_ptr(), B,
                    int(max_seqlen_q), total_q, num_pages, page_size, block_table.shape[1], Hq, Hkv, d,
                    int(bool(causal)), float(scale), int(num_splits), stream)
        else:
            rc = fn(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(), lse.data_ptr(),
                    cu_seqlens_q.data_ptr(), seqused_k.data_ptr(), block_table.data_ptr(), B, int(max_seqlen_q),
                    total_q, num_pages, page_size, block_table.shape[1], Hq, Hkv, d, int(bool(causal)),
                    float(scale), stream)
    if rc != 0:
        _raise(rc)
    return out, lse
