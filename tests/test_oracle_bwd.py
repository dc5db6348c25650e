"""Pins for the backward oracle (gradients of sum(O * dO) w.r.t. q, k, v)."""

import numpy as np
import pytest
import torch

from oracle import attention_bwd_ref, attention_ref


def _rand(B, N, Hq, Hkv, d, seed, Nk=None):
    rng = np.random.default_rng(seed)
    Nk = N if Nk is None else Nk
    return (rng.standard_normal((B, N, Hq, d)), rng.standard_normal((B, Nk, Hkv, d)),
            rng.standard_normal((B, Nk, Hkv, d)), rng.standard_normal((B, N, Hq, d)))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("hkv", [4, 2, 1])
@pytest.mark.parametrize("scale", [0.37, -0.37], ids=["pos", "neg"])
def test_matches_torch_autograd_fp64(causal, hkv, scale):
    q, k, v, do = _rand(2, 9, 4, hkv, 6, 1)
    dq, dk, dv = attention_bwd_ref(q, k, v, do, causal, scale)
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3).requires_grad_(True) for x in (q, k, v))
    # torch's math path multiplies q and k by sqrt(scale) each: a negative scale goes in as
    # |scale| with -q (the same scores); the chain rule then flips the sign of dq
    sgn = 1.0 if scale > 0 else -1.0
    out = torch.nn.functional.scaled_dot_product_attention(sgn * tq, tk, tv, is_causal=causal, scale=abs(scale),
                                                           enable_gqa=hkv != 4)
    out.backward(torch.from_numpy(do).permute(0, 2, 1, 3))
    for mine, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(mine, t.grad.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_central_finite_differences(causal):
    # d/dx sum(O * dO) by central differences on a few coordinates of q, k and v
    q, k, v, do = _rand(1, 5, 2, 1, 3, 2)
    scale, eps = 0.8, 1e-6
    dq, dk, dv = attention_bwd_ref(q, k, v, do, causal, scale)
    f = lambda qq, kk, vv: float((attention_ref(qq, kk, vv, causal, scale)[0] * do).sum())
    rng = np.random.default_rng(0)
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(6):
            idx = tuple(int(rng.integers(0, s)) for s in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            num = (f(*args_p) - f(*args_m)) / (2 * eps)
            assert abs(num - g[idx]) < 1e-7, (name, idx, num, g[idx])


def test_uniform_attention_closed_form():
    # q = 0: P is uniform 1/Nk, so dV_j = (1/Nk) sum_i dO_i and dQ, dK follow from dS.
    _, k, v, do = _rand(1, 7, 1, 1, 4, 3)
    q = np.zeros((1, 7, 1, 4))
    dq, dk, dv = attention_bwd_ref(q, k, v, do, False, 1.0)
    np.testing.assert_allclose(dv[0, :, 0], np.broadcast_to(do[0, :, 0].sum(0) / 7, (7, 4)), atol=1e-14)
    np.testing.assert_allclose(dk, 0.0, atol=1e-14)  # dS rows sum to 0 and q = 0
    # dQ_i = sum_j P_ij (dP_ij - D_i) K_j with P_ij = 1/7
    dP = do[0, :, 0] @ v[0, :, 0].T
    dS = (dP - dP.mean(1, keepdims=True)) / 7
    np.testing.assert_allclose(dq[0, :, 0], dS @ k[0, :, 0], atol=1e-13)


def test_value_gradient_is_independent_of_v_and_sums_to_dout():
    # rows of P sum to 1: sum_j dV_j = sum_i dO_i, whatever v is
    q, k, v, do = _rand(2, 8, 2, 2, 5, 4)
    for vv in (v, 3 * v - 1):
        _, _, dv = attention_bwd_ref(q, k, vv, do, True, 0.5)
        np.testing.assert_allclose(dv.sum(1), do.sum(1), atol=1e-12)
