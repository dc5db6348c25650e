"""Error model of the fp8 (e4m3) forward pass, shared by its GPU parity test and by the CPU
test that plants one-row mistakes into an emulated output (test infrastructure only).

S = Q K^T: the e4m3 products are exact, but gfx950's fp8 MFMA sums each group of 64 of them
with fewer bits than fp32. This is a property of that matrix core, measured on it with a
rounding probe (512 x 1024 MFMA outputs against exact sums, operands spread like quantised
N(0,1) data): at most 2^-14.3 of sum |q k|. Each score is allowed twice that,
    delta_j = U_S * |scale| * sum_d |q_d k_jd|,   U_S = 2^-13,
and the GPU test with one key per row (where LSE = scale q.k exactly) checks the kernel
against this allowance directly. A score error moves the LSE by at most max_j delta_j and
each weight by a factor within exp(+-delta_j). The weights p enter P V rounded to e4m3,
whose error is at most err = max(2^-4 p, min(p, 2^-10)) (3 mantissa bits; below 2^-6 the
format is subnormal with spacing 2^-9), in units where the row's largest weight is 1 (the
kernel's running max can only make its weights larger, so this is the worst case). O is
normalised by the sum of the rounded weights. Per output element:

  worst case   |O - O_ref| <= sum_j err_j |V_jd - O_ref_d| / sum_j (p_j - err_j)   (wc)
                              + sum_j p_j expm1(delta_j) |V_jd - O_ref_d| / sum_j (p_j - err_j)   (dterm)
                              + 2 half-ulps of bf16(O_ref) + 1e-4 (fp32 accumulation);
  statistical  |O - O_ref| <= K_SD * sd + dterm + 2 half-ulps + 1e-4, where
               sd = sqrt(sum_j err_j^2 |V_jd - O_ref_d|^2 / 3) / sum_j p_j
               is the spread of independent rounding errors uniform in [-err_j, err_j]
               and K_SD = 6 is fixed in advance.

Each element is held to the smaller of the two limits. At long sequences the worst case
(every rounding pointing the same way) exceeds |O| itself and the statistical limit is the one
that bites; at a few keys the worst case is the tighter one. The RMS of the error over all
checked elements must also stay below 1.5x the RMS of the predicted spread (with the bf16
output rounding, half-ulp^2 / 3). LSE: |LSE - LSE_ref| <= 1e-3 + max_j delta_j per row.
"""

import numpy as np

LSE_MAX = 1e-3
U = 2.0 ** -4
U_S = 2.0 ** -13  # fp8 MFMA accumulation allowance, relative to sum |q k|
K_SD = 6.0


def bound(qd, kd, vd, o_ref, causal, scale, rows, hkv_of):
    """Model terms for rows `rows` of every (b, h), each shaped like o_ref[b, rows, h, :]
    ([B, R, Hq, d]): (wc, dterm, sd) and the per-row LSE allowance max_j delta_j ([B, Hq, R])."""
    B, _, Hq, d = qd.shape
    R = len(rows)
    wc = np.zeros((B, R, Hq, d))
    dterm = np.zeros((B, R, Hq, d))
    sd = np.zeros((B, R, Hq, d))
    dl = np.zeros((B, Hq, R))
    j = np.arange(kd.shape[1])
    for b in range(B):
        for h in range(Hq):
            kvh = hkv_of(h)
            s = scale * (qd[b, rows, h, :] @ kd[b, :, kvh, :].T)
            delta = U_S * abs(scale) * (np.abs(qd[b, rows, h, :]) @ np.abs(kd[b, :, kvh, :]).T)
            if causal:
                vis = j[None, :] <= np.asarray(rows)[:, None]
                s = np.where(vis, s, -np.inf)
                delta = np.where(vis, delta, 0.0)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            err = np.maximum(U * p, np.minimum(p, 2.0 ** -10))
            den = (p - err).sum(axis=1)
            dev = np.abs(vd[b, None, :, kvh, :] - o_ref[b, :, h, None, :])   # [R, Nk, d]
            wc[b, :, h, :] = (err[:, :, None] * dev).sum(axis=1) / den[:, None]
            dterm[b, :, h, :] = ((p * np.expm1(delta))[:, :, None] * dev).sum(axis=1) / den[:, None]
            sd[b, :, h, :] = np.sqrt(((err * err)[:, :, None] * (dev * dev)).sum(axis=1) / 3) / p.sum(axis=1)[:, None]
            dl[b, h, :] = delta.max(axis=1)
    return wc, dterm, sd, dl


def check(og, lg, O_ref, L_ref, terms):
    """Apply the limits. og, O_ref: [B, R, Hq, d]; lg, L_ref: [B, Hq, R]; terms from bound().
    Returns (ok, figures) where figures is a dict of the measured ratios."""
    wc, dterm, sd, dl = terms
    if not (np.isfinite(og).all() and np.isfinite(lg).all()):
        return False, {"finite": False}
    half_ulp = 0.5 * np.exp2(np.floor(np.log2(np.maximum(np.abs(O_ref), 2.0 ** -126))) - 7)
    err = np.abs(og - O_ref)
    base = dterm + 2 * half_ulp + 1e-4
    lim = np.minimum(wc + base, K_SD * sd + base)
    ratio = float((err / lim).max())
    rms = float(np.sqrt((err * err).mean()))
    rms_pred = float(np.sqrt((sd * sd + half_ulp * half_ulp / 3).mean()))
    lratio = float((np.abs(lg - L_ref) / (LSE_MAX + dl)).max())
    fig = {"finite": True, "o_max": float(err.max()), "o_mean": float(err.mean()),
           "lim_max": float(lim.max()), "lim_mean": float(lim.mean()), "ratio": ratio,
           "rms": rms, "rms_pred": rms_pred, "rms_ratio": rms / rms_pred,
           "lse_max": float(np.abs(lg - L_ref).max()), "lse_ratio": lratio}
    ok = ratio <= 1.0 and rms <= 1.5 * rms_pred and lratio <= 1.0
    return ok, fig
