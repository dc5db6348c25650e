"""Planted mistakes: each mutant of the oracle (made by editing its source text on the
CPU) must be rejected by at least one pin. This shows the pins are not vacuous."""

import inspect
import json
import math
import os
import types

import numpy as np
import pytest
import torch

import oracle.attention as ref_mod

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")

MUTANTS = {
    "mask_includes_diagonal": ("S[np.arange(Nk)[None, :] > qi[:, None]]", "S[np.arange(Nk)[None, :] >= qi[:, None]]"),
    "mask_transposed": ("S[np.arange(Nk)[None, :] > qi[:, None]]", "S[np.arange(Nk)[None, :] < qi[:, None]]"),
    "scale_dropped": ("S = scale * (Qh @ Kh.T)", "S = (Qh @ Kh.T)"),
    "gqa_modulo_map": ("return h // (hq // hkv)", "return h % hkv"),
    "no_normalisation": ("Oh = (P @ Vh) / l", "Oh = (P @ Vh)"),
    "lse_without_max": ("lse = m[:, 0] + np.log(l[:, 0])", "lse = np.log(l[:, 0])"),
    "lse_log2": ("lse = m[:, 0] + np.log(l[:, 0])", "lse = m[:, 0] + np.log2(l[:, 0])"),
    "keys_transposed_in_pv": ("Oh = (P @ Vh) / l", "Oh = (P @ Vh[::-1]) / l"),
}


def _mutant(old, new):
    src = inspect.getsource(ref_mod)
    assert old in src, old
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _pins_pass(mod):
    """Run a subset of the pins against a module; True if all hold."""
    ev = lambda e: eval(e, {"__builtins__": {}}, {"e": math.e, "ln": math.log})
    try:
        for c in json.load(open(GOLDEN))["cases"]:
            q, k, v = (np.array(c[x], dtype=np.float64)[None, :, None, :] for x in "qkv")
            for causal in (False, True):
                exp = c["causal" if causal else "noncausal"]
                O, L = mod.attention_ref(q, k, v, causal, c["scale"])
                np.testing.assert_allclose(O[0, :, 0], [[ev(x) for x in r] for r in exp["O"]], atol=1e-12)
                np.testing.assert_allclose(L[0, 0], [ev(x) for x in exp["LSE"]], atol=1e-12)
        rng = np.random.default_rng(0)
        q, k, v = (rng.standard_normal(s) for s in [(1, 8, 4, 4), (1, 8, 2, 4), (1, 8, 2, 4)])
        for causal in (False, True):
            O, _ = mod.attention_ref(q, k, v, causal, 0.5)
            t = torch.nn.functional.scaled_dot_product_attention(
                *(torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k, v)), is_causal=causal, scale=0.5,
                enable_gqa=True)
            np.testing.assert_allclose(O, t.permute(0, 2, 1, 3).numpy(), atol=1e-12)
    except AssertionError:
        return False
    return True


def test_unmutated_oracle_passes():
    assert _pins_pass(ref_mod)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    assert not _pins_pass(_mutant(*MUTANTS[name])), f"pins did not catch mutant {name}"
