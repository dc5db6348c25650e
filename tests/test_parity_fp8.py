"""GPU parity of the fp8 (e4m3) forward pass (fa_fwd_fp8) against the fp64 oracle.

Inputs: seeded N(0,1) draws quantised per tensor to e4m3 (scale = amax / 224, so no value
saturates); the oracle runs on the dequantised values (scale * e4m3 value, exact in fp64).

Tolerance, derived from the arithmetic (the pages give none for FP8). S = Q K^T: the e4m3
products are exact, but gfx950's fp8 MFMA sums each group of 64 of them with fewer bits than
fp32 - measured on the GPU with operands like these (N(0,1) draws quantised with amax/224, 512
trials of 1024 outputs): at most 2^-14.3 of sum |q k|. Each score is allowed an error of
    delta_j = U_S * scale * sum_d |q_d k_jd|,   U_S = 2^-13
(twice the worst measured), which moves the LSE by at most max_j delta_j and each weight by a
factor within exp(+-delta_j). The weights p enter P V rounded to e4m3, whose error is at most
err = max(2^-4 * p, min(p, 2^-10)) (3 mantissa bits; below 2^-6 the format is subnormal with
spacing 2^-9), in units where the row's largest weight is 1 (the kernel's running max can
only make its weights larger, so this is the worst case). O is normalised by the sum of the
rounded weights, so for every output element
    |O - O_ref| <= sum_j (err_j + p_j (exp(delta_j) - 1)) |V_jd - O_ref_d| / sum_j (p_j - err_j)
plus one bf16 ulp of O_ref (the output rounding, with room for a result that crosses into
the next binade) and 1e-4 for fp32 accumulation. At long sequences this worst
case (every rounding error pointing the same way) exceeds |O| itself, so the RMS of the error
is also checked against the spread that independent roundings give: a rounding error
uniform in [-err_j, err_j] has variance err_j^2 / 3, so
    sd(O_d) = sqrt(sum_j err_j^2 |V_jd - O_ref_d|^2 / 3) / sum_j p_j,
combined with the bf16 output rounding (half-ulp^2 / 3); the RMS error over all checked
elements must stay below 1.5x the RMS of that prediction (a wrong V column, weight or
normalisation misses it by an order of magnitude or more). The LSE uses the fp32 sum of the
unrounded weights: |LSE - LSE_ref| <= 1e-3 + max_j delta_j per row.
"""

import numpy as np
import pytest
import torch

import exact_attention_06_amd as fa
from exact_attention_06_amd import workloads as W
from oracle import attention_ref

pytestmark = pytest.mark.gpu

LSE_MAX = 1e-3
U = 2.0 ** -4
U_S = 2.0 ** -13  # fp8 MFMA accumulation, relative to sum |q k| (see the module docstring)


def _say(msg):
    print(msg, flush=True)


def _quant(x):
    s = float(x.abs().max()) / 224.0
    return (x / s).to(torch.float8_e4m3fn), s


def _bound(qd, kd, vd, o_ref, causal, scale, rows, hkv_of):
    """Per-element worst-case bound and predicted spread for rows `rows` of every (b, h),
    each shaped like o_ref[b, rows, h, :], and the per-row LSE allowance max_j delta_j
    ([B, Hq, R])."""
    B, _, Hq, d = qd.shape
    out = np.zeros((B, len(rows), Hq, d))
    sd = np.zeros((B, len(rows), Hq, d))
    dl = np.zeros((B, Hq, len(rows)))
    j = np.arange(kd.shape[1])
    for b in range(B):
        for h in range(Hq):
            kvh = hkv_of(h)
            s = scale * (qd[b, rows, h, :] @ kd[b, :, kvh, :].T)
            delta = U_S * scale * (np.abs(qd[b, rows, h, :]) @ np.abs(kd[b, :, kvh, :]).T)
            if causal:
                vis = j[None, :] <= np.asarray(rows)[:, None]
                s = np.where(vis, s, -np.inf)
                delta = np.where(vis, delta, 0.0)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            err = np.maximum(U * p, np.minimum(p, 2.0 ** -10))
            den = (p - err).sum(axis=1)
            dev = np.abs(vd[b, None, :, kvh, :] - o_ref[b, :, h, None, :])   # [R, Nk, d]
            tot = err + p * np.expm1(delta)
            out[b, :, h, :] = (tot[:, :, None] * dev).sum(axis=1) / den[:, None]
            sd[b, :, h, :] = np.sqrt(((err * err)[:, :, None] * (dev * dev)).sum(axis=1) / 3) / p.sum(axis=1)[:, None]
            dl[b, h, :] = delta.max(axis=1)
    return out, sd, dl


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
    bound, sd, dl = _bound(qd, kd, vd, O_ref, causal, scale, rows, lambda h: h // g)
    og = o.float().cpu().numpy().astype(np.float64)[:, rows]
    lg = lse.cpu().numpy().astype(np.float64)[:, :, rows]
    assert np.isfinite(og).all() and np.isfinite(lg).all(), f"{name}: non-finite output"
    half_ulp = 0.5 * np.exp2(np.floor(np.log2(np.maximum(np.abs(O_ref), 2.0 ** -126))) - 7)
    err = np.abs(og - O_ref)
    lim = bound + 2 * half_ulp + 1e-4
    ratio = float((err / lim).max())
    rms = float(np.sqrt((err * err).mean()))
    rms_pred = float(np.sqrt((sd * sd + half_ulp * half_ulp / 3).mean()))
    lerr = float(np.abs(lg - L_ref).max())
    lratio = float((np.abs(lg - L_ref) / (LSE_MAX + dl)).max())
    _say(f"  {name}: O max err {err.max():.3e} mean {err.mean():.3e} | bound max {bound.max():.3e} "
         f"mean {bound.mean():.3e} | worst err/limit {ratio:.3f} | RMS {rms:.3e} vs predicted "
         f"{rms_pred:.3e} | LSE max {lerr:.3e} (worst share of 1e-3 + allowance {lratio:.3f})")
    assert ratio <= 1.0, f"{name}: error above the fp8 bound (ratio {ratio:.3f})"
    assert rms <= 1.5 * rms_pred, f"{name}: RMS error {rms:.3e} above 1.5x the predicted {rms_pred:.3e}"
    assert lratio <= 1.0, f"{name}: LSE max {lerr:.3e} above 1e-3 + the score allowance (ratio {lratio:.3f})"


SMALL = [
    # name,        B,  N,    Hq, Hkv, d,  seed
    ("tiny",       1,  256,  2,  2,  128, 101),
    ("ragged",     1,  257,  8,  8,  128, 102),
    ("gqa_tail",   2,  300,  4,  2,  128, 103),
    ("hd256",      1,  300,  2,  1,  256, 104),
    ("few",        1,  3,    2,  1,  128, 105),
    ("mid",        1,  1024, 4,  4,  256, 106),
]


@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_fp8_all_rows(case, causal):
    name, B, N, Hq, Hkv, d, seed = case
    _run(name, B, N, Hq, Hkv, d, causal, seed)


@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
@pytest.mark.parametrize("wname", ["hd128_N8192_mha", "hd256_N8192"])
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
