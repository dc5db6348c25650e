"""Planted mistakes in the backward oracle: each mutant of attention_bwd_ref (made by
editing its source text on the CPU) must be rejected by the backward pins (torch autograd
in float64, central finite differences of the forward oracle, the closed forms). This shows
those pins are not vacuous."""

import inspect
import types

import numpy as np
import pytest
import torch

import oracle.attention as ref_mod

MUTANTS = {
    "ds_sign_flipped": ("dS = P * (dP - D)", "dS = P * (D - dP)"),
    "d_term_dropped": ("dS = P * (dP - D)", "dS = P * dP"),
    "dq_scale_dropped": ("dq[b, :, h, :] = scale * (dS @ Kh)", "dq[b, :, h, :] = dS @ Kh"),
    "dk_untransposed_ds": ("dk[b, :, kvh, :] += scale * (dS.T @ Qh)", "dk[b, :, kvh, :] += scale * (dS @ Qh)"),
    "dv_group_overwritten": ("dv[b, :, kvh, :] += P.T @ dOh", "dv[b, :, kvh, :] = P.T @ dOh"),
    "dk_group_overwritten": ("dk[b, :, kvh, :] += scale * (dS.T @ Qh)", "dk[b, :, kvh, :] = scale * (dS.T @ Qh)"),
    "p_unnormalised": ("P /= P.sum(axis=1, keepdims=True)", "P /= P.sum(axis=0, keepdims=True)"),
    "dp_uses_k": ("dP = dOh @ Vh.T", "dP = dOh @ Kh.T"),
    "mask_transposed": ("S[np.arange(Nk)[None, :] > np.arange(Nq)[:, None]] = -np.inf",
                        "S[np.arange(Nk)[None, :] < np.arange(Nq)[:, None]] = -np.inf"),
}


def _mutant(old, new):
    src = inspect.getsource(ref_mod)
    assert src.count(old) >= 1, old
    # only the backward function is edited: its text follows "def attention_bwd_ref"
    head, tail = src.split("def attention_bwd_ref", 1)
    assert old in tail, old
    mod = types.ModuleType("oracle_bwd_mutant")
    exec(compile(head + "def attention_bwd_ref" + tail.replace(old, new), "oracle_bwd_mutant", "exec"),
         mod.__dict__)
    return mod


def _rand(B, N, Hq, Hkv, d, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, N, Hq, d)), rng.standard_normal((B, N, Hkv, d)),
            rng.standard_normal((B, N, Hkv, d)), rng.standard_normal((B, N, Hq, d)))


def _pins_pass(mod):
    """The backward pins against a module: autograd of torch's fp64 SDPA (MHA and GQA, causal
    and not) and central differences of the (unmutated) forward oracle."""
    try:
        for causal in (False, True):
            for hkv in (4, 2):
                q, k, v, do = _rand(2, 9, 4, hkv, 6, 1)
                scale = 0.37
                dq, dk, dv = mod.attention_bwd_ref(q, k, v, do, causal, scale)
                tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3).requires_grad_(True) for x in (q, k, v))
                out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale,
                                                                       enable_gqa=hkv != 4)
                out.backward(torch.from_numpy(do).permute(0, 2, 1, 3))
                for mine, t in ((dq, tq), (dk, tk), (dv, tv)):
                    np.testing.assert_allclose(mine, t.grad.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-12)
        q, k, v, do = _rand(1, 5, 2, 1, 3, 2)
        eps = 1e-6
        dq, dk, dv = mod.attention_bwd_ref(q, k, v, do, True, 0.8)
        f = lambda qq, kk, vv: float((ref_mod.attention_ref(qq, kk, vv, True, 0.8)[0] * do).sum())
        for x, g, pos in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
            for idx in ((0, 1, 0, 2), (0, 3, 0, 1)):
                if idx[2] >= x.shape[2]:
                    continue
                xp, xm = x.copy(), x.copy()
                xp[idx] += eps
                xm[idx] -= eps
                a_p, a_m = [q, k, v], [q, k, v]
                a_p[pos], a_m[pos] = xp, xm
                num = (f(*a_p) - f(*a_m)) / (2 * eps)
                assert abs(num - g[idx]) < 1e-7
    except AssertionError:
        return False
    return True


def test_unmutated_backward_oracle_passes():
    assert _pins_pass(ref_mod)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_backward_mutant_is_caught(name):
    assert not _pins_pass(_mutant(*MUTANTS[name])), f"backward pins did not catch mutant {name}"
