"""The allocation-free backward entry point (fa_bwd_noalloc, through the C ABI) against
fa_bwd on the same inputs: the same kernels with D in the library's fixed device scratch
instead of a caller workspace, so the gradients must agree bit for bit. Two calls in a row,
the second on a smaller problem (the scratch keeps the first call's D, which the second
must not depend on)."""

import ctypes

import pytest
import torch

from exact_attention_06_amd import _lib
from exact_attention_06_amd import workloads as W

pytestmark = pytest.mark.gpu


def _grads_both_ways(B, N, Hq, Hkv, d, causal, seed):
    lib = _lib.load()
    q, k, v = (t.cuda() for t in W.make_qkv(B, N, N, Hq, Hkv, d, seed))
    g = torch.Generator().manual_seed(seed + 7)
    do = torch.randn((B, N, Hq, d), generator=g).to(torch.bfloat16).cuda()
    scale = float(torch.tensor(d ** -0.5, dtype=torch.float32))
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    assert lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, N, N, Hq, Hkv, d,
                      int(causal), ctypes.c_float(scale), st) == 0
    ref = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
    nbytes = int(lib.fa_bwd_workspace_bytes(B, N, Hq))
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    assert lib.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                      ref[0].data_ptr(), ref[1].data_ptr(), ref[2].data_ptr(), ws.data_ptr(), nbytes, B, N, N, Hq,
                      Hkv, d, int(causal), ctypes.c_float(scale), st) == 0
    got = [torch.full_like(q, float("nan")), torch.full_like(k, float("nan")), torch.full_like(v, float("nan"))]
    assert lib.fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                              do.data_ptr(), got[0].data_ptr(), got[1].data_ptr(), got[2].data_ptr(), B, N, N, Hq,
                              Hkv, d, int(causal), ctypes.c_float(scale), st) == 0
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_backward_equals_workspace_backward_twice():
    for case in ((2, 700, 8, 2, 128, True, 301), (1, 300, 4, 4, 256, False, 302)):
        print(f"[gpu] fa_bwd_noalloc vs fa_bwd {case}", flush=True)
        ref, got = _grads_both_ways(*case)
        for name, a, b in zip(("dq", "dk", "dv"), ref, got):
            assert torch.isfinite(b.float()).all(), name
            assert torch.equal(a, b), f"{case} {name}: max diff {(a.float() - b.float()).abs().max().item()}"
