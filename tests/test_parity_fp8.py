"""GPU parity of the fp8 (e4m3) forward pass (fa_fwd_fp8) against the fp64 oracle.

Inputs: seeded N(0,1) draws quantised per tensor to e4m3 (scale = amax / 224, so no value
saturates); the oracle runs on the dequantised values (scale * e4m3 value, exact in fp64).

Tolerance, derived from the arithmetic (the pages give none for FP8): the error model of
tests/fp8_bound.py - the fp8 MFMA's score accumulation allowance (a measured gfx950 property,
checked directly by test_fp8_score_accumulation_within_allowance), the e4m3 rounding of P,
normalisation by the sum of the rounded weights, and the bf16 output rounding. Every checked
element is held to the smaller of a worst-case limit and a statistical one (6 standard
deviations of independent roundings, fixed in advance), and the RMS error to 1.5x the
predicted spread; the LSE to 1e-3 plus the score allowance.
"""

import numpy as np
import pytest
import torch

import exact_attention_06_amd as fa
from exact_attention_06_amd import workloads as W
from oracle import attention_ref

from fp8_bound import U_S, bound, check

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _quant(x):
    s = float(x.abs().max()) / 224.0
    return (x / s).to(torch.float8_e4m3fn), s


def _run(name, B, N, Hq, Hkv, d, causal, seed, rows=None, Nk=None, scale=None):
    Nk = N if Nk is None else Nk
    q, k, v = W.make_qkv(B, N, Nk, Hq, Hkv, d, seed, dtype=torch.float32)
    (q8, qs), (k8, ks), (v8, vs) = _quant(q), _quant(k), _quant(v)
    if scale is None:
        scale = float(torch.tensor(d ** -0.5, dtype=torch.float32))
    _say(f"[gpu] fp8 {name} B={B} Nq={N} Nk={Nk} Hq={Hq} Hkv={Hkv} d={d} causal={causal} scale={scale} seed={seed}")
    o, lse = fa.forward_fp8(q8.cuda(), k8.cuda(), v8.cuda(), qs, ks, vs, causal=causal, scale=scale)
    torch.cuda.synchronize()
    qd = q8.double().numpy() * qs
    kd = k8.double().numpy() * ks
    vd = v8.double().numpy() * vs
    rows = np.arange(N) if rows is None else np.asarray(sorted(set(int(r) for r in rows)))
    O_ref, L_ref = attention_ref(qd, kd, vd, causal, scale, rows=rows)     # [B, Hq, R, d], [B, Hq, R]
    O_ref = O_ref.transpose(0, 2, 1, 3)                                    # [B, R, Hq, d]
    g = Hq // Hkv
    terms = bound(qd, kd, vd, O_ref, causal, scale, rows, lambda h: h // g)
    og = o.float().cpu().numpy().astype(np.float64)[:, rows]
    lg = lse.cpu().numpy().astype(np.float64)[:, :, rows]
    ok, f = check(og, lg, O_ref, L_ref, terms)
    assert f["finite"], f"{name}: non-finite output"
    _say(f"  {name}: O max err {f['o_max']:.3e} mean {f['o_mean']:.3e} | limit max {f['lim_max']:.3e} "
         f"mean {f['lim_mean']:.3e} | worst err/limit {f['ratio']:.3f} | RMS {f['rms']:.3e} vs predicted "
         f"{f['rms_pred']:.3e} ({f['rms_ratio']:.2f}x) | LSE max {f['lse_max']:.3e} (worst share of 1e-3 + "
         f"allowance {f['lse_ratio']:.3f})")
    assert ok, f"{name}: outside the fp8 error model {f}"


SMALL = [
    # name,        B,  N,    Hq, Hkv, d,  seed
    ("tiny",       1,  256,  2,  2,  128, 101),
    ("ragged",     1,  257,  8,  8,  128, 102),
    ("gqa_tail",   2,  300,  4,  2,  128, 103),
    ("hd256",      1,  300,  2,  1,  256, 104),
    ("few",        1,  3,    2,  1,  128, 105),
    ("mid",        1,  1024, 4,  4,  256, 106),
    # hd128 runs a software-pipelined tile loop: GQA over many main tiles, and an odd count
    # of main tiles (31) followed by a 16-key tail tile
    ("gqa_mid",    2,  1536, 8,  2,  128, 111),
    ("long_odd",   1,  2000, 2,  1,  128, 112),
]


@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_fp8_all_rows(case, causal):
    name, B, N, Hq, Hkv, d, seed = case
    _run(name, B, N, Hq, Hkv, d, causal, seed)


@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
@pytest.mark.parametrize("wname", ["hd128_N8192_mha", "hd128_N8192_gqa4", "hd256_N8192"])
def test_fp8_full_size_sampled_rows(wname, causal):
    w = W.by_name(wname)
    rows = [0, 1, 63, 64, 127, 128, 4095, 4096, w.N - 2, w.N - 1] + list(range(200, 8000, 1201))
    _run(wname, w.B, w.N, w.Hq, w.Hkv, w.d, causal, w.seed, rows=rows)


RECT = [
    # name,        Nq,  Nk,  Hq, Hkv, d,  seed
    ("q_short",    70,  900, 2,  1,  128, 108),
    ("q_long",     300, 65,  4,  4,  256, 109),
    ("k_single",   129, 1,   2,  1,  128, 110),
]


@pytest.mark.parametrize("case", RECT, ids=[c[0] for c in RECT])
def test_fp8_rectangular_noncausal(case):
    name, Nq, Nk, Hq, Hkv, d, seed = case
    _run(name, 1, Nq, Hq, Hkv, d, False, seed, Nk=Nk)


@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
@pytest.mark.parametrize("d", [128, 256])
def test_fp8_zero_scale(d, causal):
    # every visible key gets weight 1 exactly (in e4m3 too): O = mean of the visible V rows
    _run(f"zero_scale_d{d}", 1, 257, 2, 1, d, causal, 111 + d, scale=0.0)


@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
@pytest.mark.parametrize("d", [128, 256])
def test_fp8_negative_scale(d, causal):
    # scale -1/sqrt(d): the kernel flips the sign bit of every e4m3 Q byte (exact)
    _run(f"neg_scale_d{d}", 2, 600, 4, 2, d, causal, 140 + d, scale=-float(d) ** -0.5)


@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
@pytest.mark.parametrize("d", [128, 256])
def test_fp8_hot_scores(d, causal):
    # scale 1: nearly one-hot rows, the running max jumps far past the rescale threshold
    _run(f"hot_scores_d{d}", 1, 600, 2, 1, d, causal, 120 + d, scale=1.0)


@pytest.mark.parametrize("d", [128, 256])
def test_fp8_score_accumulation_within_allowance(d):
    # one key per row: LSE = scale * q.k exactly, so the kernel's LSE exposes the fp8 MFMA's
    # accumulation error on the score itself; it must stay within the allowance U_S used above
    B, Nq, H = 2, 4096, 8
    q, k, v = W.make_qkv(B, Nq, 1, H, H, d, 130 + d, dtype=torch.float32)
    (q8, qs), (k8, ks), (v8, vs) = _quant(q), _quant(k), _quant(v)
    scale = 1.0
    _say(f"[gpu] fp8 score accumulation d={d} B={B} Nq={Nq} Hq={H} Nk=1")
    _, lse = fa.forward_fp8(q8.cuda(), k8.cuda(), v8.cuda(), qs, ks, vs, scale=scale)
    torch.cuda.synchronize()
    qd = q8.double().numpy() * qs                       # [B, Nq, H, d]
    kd = k8.double().numpy() * ks                       # [B, 1, H, d]
    exact = scale * np.einsum("bnhd,bhd->bhn", qd, kd[:, 0])
    mag = scale * np.einsum("bnhd,bhd->bhn", np.abs(qd), np.abs(kd[:, 0]))
    err = np.abs(lse.cpu().numpy().astype(np.float64) - exact)
    ratio = err / (U_S * mag + 1e-6 * np.abs(exact) + 1e-7)
    _say(f"  max |LSE - s| {err.max():.3e}, max error / sum|q k| {float((err / mag).max()):.3e} "
         f"(2^{np.log2(float((err / mag).max())):.1f}), worst share of the allowance {float(ratio.max()):.3f}")
    assert float(ratio.max()) <= 1.0


def test_fp8_scales_enter_exactly():
    # doubling v_scale doubles O (exactly, up to the bf16 output rounding: both are rounded
    # from the same fp32 value times 2)
    q, k, v = W.make_qkv(1, 300, 300, 2, 2, 128, 107, dtype=torch.float32)
    (q8, qs), (k8, ks), (v8, vs) = _quant(q), _quant(k), _quant(v)
    o1, l1 = fa.forward_fp8(q8.cuda(), k8.cuda(), v8.cuda(), qs, ks, vs)
    o2, l2 = fa.forward_fp8(q8.cuda(), k8.cuda(), v8.cuda(), qs, ks, 2 * vs)
    torch.cuda.synchronize()
    assert torch.equal(o2, 2 * o1) and torch.equal(l1, l2)


def test_fp8_repeated_full_size_launches_are_bitwise_equal():
    # every wave reads every wave's share of each K/V tile: launches must agree bit for bit
    w = W.by_name("hd256_N8192")
    g = torch.Generator(device="cuda")
    g.manual_seed(w.seed)
    x = [torch.randn((w.B, w.N, h, w.d), generator=g, device="cuda") for h in (w.Hq, w.Hkv, w.Hkv)]
    (q8, qs), (k8, ks), (v8, vs) = (_quant(t) for t in x)
    for causal in (False, True):
        _say(f"[gpu] fp8 repeated launches causal={causal}")
        o0, l0 = fa.forward_fp8(q8, k8, v8, qs, ks, vs, causal=causal, scale=w.scale)
        for _ in range(2):
            o1, l1 = fa.forward_fp8(q8, k8, v8, qs, ks, vs, causal=causal, scale=w.scale)
            torch.cuda.synchronize()
            assert torch.equal(o0, o1) and torch.equal(l0, l1)
