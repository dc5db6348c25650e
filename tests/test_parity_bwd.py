"""GPU parity of the backward pass (dq, dk, dv through the C ABI) against the fp64 oracle.

The inputs q, k, v, dout are the same bf16/fp16 values on both sides; the GPU's o and lse
come from its own forward pass (as in training). P and dS enter the MFMAs rounded to the
input type, and the gradients are rounded to it on output, so the bound is relative to the
gradient's own scale: per tensor, max-abs error <= 1e-2 * max|ref| and mean-abs error <=
5e-3 * mean|ref|. Rounding a value to bf16 alone costs up to 2^-9 (1.95e-3) of it and 2^-10
on average; measured ratios are 2e-3..5.4e-3 (max) and 1.9e-3..3.8e-3 (mean) for bf16 and
about ten times smaller for fp16. The measured errors are printed for every case.
"""

import numpy as np
import pytest
import torch

import exact_attention_06_amd as fa
from exact_attention_06_amd import workloads as W
from oracle import attention_bwd_ref

pytestmark = pytest.mark.gpu

MAX_REL, MEAN_REL = 1e-2, 5e-3


def _say(msg):
    print(msg, flush=True)


def _compare(name, got_all, ref_all):
    for tname, got, ref in zip(("dq", "dk", "dv"), got_all, ref_all):
        got = got.float().cpu().numpy().astype(np.float64)
        assert np.isfinite(got).all(), f"{name}/{tname}: non-finite"
        err = np.abs(got - ref)
        mx, mean, rmax, rmean = err.max(), err.mean(), np.abs(ref).max(), np.abs(ref).mean()
        _say(f"  {name}/{tname}: max err {mx:.3e} (max|ref| {rmax:.3e}, ratio {mx / max(rmax, 1e-300):.2e}) "
             f"mean err {mean:.3e} (mean|ref| {rmean:.3e}, ratio {mean / max(rmean, 1e-300):.2e})")
        if rmax == 0.0:  # a gradient that is exactly zero (dq, dk at scale 0)
            assert mx == 0.0, f"{name}/{tname}"
            continue
        assert mx <= MAX_REL * rmax and mean <= MEAN_REL * rmean, f"{name}/{tname}"


def _run(name, B, Nq, Nk, Hq, Hkv, d, causal, seed, dtype=torch.bfloat16, heads=None, scale=None):
    """heads=[(b, kvh), ...]: compare only those KV heads' groups (dq of their query heads,
    their dk and dv), each against its own oracle call."""
    q, k, v = W.make_qkv(B, Nq, Nk, Hq, Hkv, d, seed, dtype=dtype)
    g = torch.Generator().manual_seed(seed + 7)
    do = torch.randn((B, Nq, Hq, d), generator=g).to(dtype)
    if scale is None:
        scale = float(torch.tensor(d ** -0.5, dtype=torch.float32))
    _say(f"[gpu] bwd {name} B={B} Nq={Nq} Nk={Nk} Hq={Hq} Hkv={Hkv} d={d} causal={causal} {dtype} scale={scale}")
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = fa.forward(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv = fa.backward(qd, kd, vd, o, lse, dod, causal=causal, scale=scale)
    torch.cuda.synchronize()
    if heads is None:
        _compare(name, (dq, dk, dv), attention_bwd_ref(q, k, v, do, causal, scale))
        return
    gsz = Hq // Hkv
    for b, kvh in heads:
        hs = slice(kvh * gsz, (kvh + 1) * gsz)
        ref = attention_bwd_ref(q[b:b + 1, :, hs], k[b:b + 1, :, kvh:kvh + 1], v[b:b + 1, :, kvh:kvh + 1],
                                do[b:b + 1, :, hs], causal, scale)
        got = (dq[b:b + 1, :, hs], dk[b:b + 1, :, kvh:kvh + 1], dv[b:b + 1, :, kvh:kvh + 1])
        _compare(f"{name}[b={b},kvh={kvh}]", got, ref)


CASES = [
    # name,           B,  Nq,   Nk,  Hq, Hkv,  d, seed
    ("tiny",          1,  256,  256,  2,  2, 128, 61),
    ("ragged",        1,  257,  257,  8,  8, 128, 62),
    ("gqa_tail",      2,  300,  300,  4,  2, 128, 63),
    ("hd256",         1,  200,  200,  2,  1, 256, 64),
    ("few",           2,    3,    3,  2,  1, 128, 65),
    ("mid",           1, 1024, 1024,  4,  4, 128, 66),
    # many key tiles that skip the mask in the dq kernel, then a ragged tail tile
    ("ragged_long",   2, 1100, 1100,  4,  4, 128, 69),
    ("gqa_long_256",  1, 1500, 1500,  8,  2, 256, 70),
]


@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bwd_full(case, causal):
    name, B, Nq, Nk, Hq, Hkv, d, seed = case
    _run(name, B, Nq, Nk, Hq, Hkv, d, causal, seed)


@pytest.mark.parametrize("case", [("rect_qk", 1, 100, 333, 2, 1, 128, 67), ("rect_kq", 1, 333, 90, 2, 2, 256, 68)],
                         ids=["rect_qk", "rect_kq"])
def test_bwd_rectangular(case):
    name, B, Nq, Nk, Hq, Hkv, d, seed = case
    _run(name, B, Nq, Nk, Hq, Hkv, d, False, seed)


@pytest.mark.parametrize("d", [128, 256])
def test_bwd_fp16(d):
    _run(f"fp16_d{d}", 1, 300, 300, 2, 1, d, True, 69 + d, dtype=torch.float16)


@pytest.mark.parametrize("d", [128, 256])
def test_bwd_zero_scale(d):
    # scale 0: P is uniform over the visible keys, dq = dk = 0 exactly, dv = P^T dO
    _run(f"zero_scale_d{d}", 1, 257, 257, 2, 1, d, True, 80 + d, scale=0.0)


FULL_BWD = [W.by_name(n) for n in ("hd128_N8192_mha", "hd128_N8192_gqa4", "hd256_N8192")]


@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
@pytest.mark.parametrize("w", FULL_BWD, ids=[w.name for w in FULL_BWD])
def test_bwd_full_size_two_heads(w, causal):
    # full-size launch; the oracle covers two KV-head groups in different batches: KV head 0
    # of the last batch and the last KV head of the first batch (with their query heads)
    _run(w.name, w.B, w.N, w.N, w.Hq, w.Hkv, w.d, causal, w.seed, heads=[(w.B - 1, 0), (0, w.Hkv - 1)])


@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
@pytest.mark.parametrize("d", [128, 256])
def test_bwd_negative_scale(d, causal):
    # scale -1/sqrt(d): scores of the opposite sign; dq = scale dS K and dk = scale dS^T Q
    # carry the sign
    _run(f"neg_scale_d{d}", 2, 300, 300, 4, 2, d, causal, 90 + d, scale=-float(d) ** -0.5)


def _random_case(i):
    g = np.random.default_rng(7000 + i)
    d = int(g.choice([128, 256]))
    hkv = int(g.choice([1, 2]))
    hq = hkv * int(g.choice([1, 2, 4]))
    causal = bool(g.integers(0, 2))
    nq = int(g.integers(1, 400))
    nk = nq if causal else int(g.integers(1, 400))
    dtype = torch.bfloat16 if g.integers(0, 3) else torch.float16
    return (f"rb{i}", int(g.integers(1, 3)), nq, nk, hq, hkv, d, causal, 8000 + i, dtype)


RB = [_random_case(i) for i in range(12)]


@pytest.mark.parametrize("case", RB, ids=[c[0] for c in RB])
def test_bwd_random_shape(case):
    name, B, Nq, Nk, Hq, Hkv, d, causal, seed, dtype = case
    _run(name, B, Nq, Nk, Hq, Hkv, d, causal, seed, dtype=dtype)


@pytest.mark.parametrize("wname", ["hd128_N8192_mha", "hd256_N8192"])
def test_bwd_repeated_full_size_launches_are_bitwise_equal(wname):
    # the backward kernels stream Q/dO and K/V tiles loaded by all waves: launches must agree
    w = W.by_name(wname)
    g = torch.Generator(device="cuda")
    g.manual_seed(w.seed)
    q, k, v, do = (torch.randn((w.B, w.N, h, w.d), generator=g, device="cuda").to(torch.bfloat16)
                   for h in (w.Hq, w.Hkv, w.Hkv, w.Hq))
    for causal in (False, True):
        _say(f"[gpu] bwd repeated launches {wname} causal={causal}")
        o, lse = fa.forward(q, k, v, causal=causal, scale=w.scale)
        r0 = fa.backward(q, k, v, o, lse, do, causal=causal, scale=w.scale)
        r1 = fa.backward(q, k, v, o, lse, do, causal=causal, scale=w.scale)
        torch.cuda.synchronize()
        for a, b in zip(r0, r1):
            assert torch.equal(a, b)
