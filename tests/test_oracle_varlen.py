"""Pins for the variable-length / seqused_k / paged-K/V oracle (oracle/varlen.py).

Each check compares the oracle with something other than itself: closed forms worked by
hand for the bottom-right causal alignment, the independently pinned dense oracle
(equal-length sequences, decode rows, chunked prefill against the full causal square),
truncated keys for seqused_k, a packed copy of a shuffled paged cache, and empty rows by
definition. Planted mutants of the module's source must each fail at least one pin.
Sources: "[RFC] FA4 - head_dim=256 & head_dim=512", section "Phase 2" (paged KV with the
page size equal to the key tile, seqused_k, varlen); the Dutch page, section
"Compatibiliteit en huidige status" (variable-length batches via cu_seqlens).
"""

import inspect
import math
import types

import numpy as np
import pytest

import oracle.varlen as vmod
from oracle import attention_ref
from oracle.varlen import attention_paged_ref, attention_varlen_ref

E = math.e


def _pack(lengths, H, d, rng):
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return cu, rng.standard_normal((int(cu[-1]), H, d))


# --- closed forms worked by hand (catch: top-left instead of bottom-right, wrong offsets)

def test_bottom_right_two_queries_three_keys():
    # scale 1, q = 1, k = (0, 1, 2), v = (1, 2, 4): scores of either row are (0, 1, 2).
    # Bottom-right: row 0 sees keys 0..1, row 1 sees keys 0..2.
    q = np.ones((2, 1, 1))
    k = np.array([0.0, 1.0, 2.0]).reshape(3, 1, 1)
    v = np.array([1.0, 2.0, 4.0]).reshape(3, 1, 1)
    O, L = attention_varlen_ref(q, k, v, [0, 2], [0, 3], True, 1.0)
    np.testing.assert_allclose(O[:, 0, 0], [(1 + 2 * E) / (1 + E), (1 + 2 * E + 4 * E * E) / (1 + E + E * E)],
                               rtol=0, atol=1e-14)
    np.testing.assert_allclose(L[0], [math.log(1 + E), math.log(1 + E + E * E)], rtol=0, atol=1e-14)
    # non-causal: both rows see all three keys
    O, L = attention_varlen_ref(q, k, v, [0, 2], [0, 3], False, 1.0)
    np.testing.assert_allclose(O[:, 0, 0], [(1 + 2 * E + 4 * E * E) / (1 + E + E * E)] * 2, rtol=0, atol=1e-14)


def test_more_queries_than_keys_leaves_empty_rows():
    # Lq = 3, Lk = 1, causal: rows 0 and 1 see no key (O = 0, LSE = -inf); row 2 sees key 0.
    q = np.array([5.0, -3.0, 0.5]).reshape(3, 1, 1)
    k = np.array([2.0]).reshape(1, 1, 1)
    v = np.array([7.0]).reshape(1, 1, 1)
    O, L = attention_varlen_ref(q, k, v, [0, 3], [0, 1], True, 0.25)
    np.testing.assert_array_equal(O[:, 0, 0], [0.0, 0.0, 7.0])
    assert L[0, 0] == -np.inf and L[0, 1] == -np.inf
    assert L[0, 2] == pytest.approx(0.25 * 0.5 * 2.0, abs=1e-15)


def test_zero_used_keys_gives_empty_rows():
    rng = np.random.default_rng(3)
    cu, q = _pack([4, 5], 2, 8, rng)
    cuk, k = _pack([6, 6], 1, 8, rng)
    v = rng.standard_normal(k.shape)
    for causal in (False, True):
        O, L = attention_varlen_ref(q, k, v, cu, cuk, causal, 0.3, seqused_k=[0, 6])
        assert np.all(O[:4] == 0) and np.all(L[:, :4] == -np.inf)
        assert np.all(np.isfinite(L[:, 4:]))


# --- against the dense oracle (pinned in test_oracle.py)

@pytest.mark.parametrize("causal", [False, True])
def test_equal_lengths_match_dense_oracle(causal):
    rng = np.random.default_rng(4)
    lens = [1, 7, 33, 64, 5]
    cu, q = _pack(lens, 4, 16, rng)
    _, k = _pack(lens, 2, 16, rng)
    v = rng.standard_normal(k.shape)
    O, L = attention_varlen_ref(q, k, v, cu, cu, causal, 0.2)
    for b, n in enumerate(lens):
        s = slice(cu[b], cu[b + 1])
        Od, Ld = attention_ref(q[None, s], k[None, s], v[None, s], causal, 0.2)
        np.testing.assert_allclose(O[s], Od[0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(L[:, s], Ld[0], rtol=0, atol=1e-13)


def test_decode_rows_see_every_key():
    # one query per sequence, causal: bottom-right lets it see all keys (= non-causal)
    rng = np.random.default_rng(5)
    klens = [1, 9, 40]
    cu = np.arange(4)
    q = rng.standard_normal((3, 2, 8))
    cuk, k = _pack(klens, 2, 8, rng)
    v = rng.standard_normal(k.shape)
    O, L = attention_varlen_ref(q, k, v, cu, cuk, True, 0.4)
    for b in range(3):
        s = slice(cuk[b], cuk[b + 1])
        Od, Ld = attention_ref(q[None, b:b + 1], k[None, s], v[None, s], False, 0.4)
        np.testing.assert_allclose(O[b], Od[0, 0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(L[:, b], Ld[0, :, 0], rtol=0, atol=1e-13)


def test_chunked_prefill_equals_rows_of_the_full_causal_square():
    # the last Lq queries of a length-Lk sequence against all Lk keys, bottom-right causal,
    # are rows Lk-Lq .. Lk-1 of the full Lk x Lk causal attention (dense, top-left)
    rng = np.random.default_rng(6)
    lk, lq = 37, 11
    qfull = rng.standard_normal((1, lk, 3, 8))
    k = rng.standard_normal((1, lk, 3, 8))
    v = rng.standard_normal((1, lk, 3, 8))
    Of, Lf = attention_ref(qfull, k, v, True, 0.35)
    O, L = attention_varlen_ref(qfull[0, lk - lq:], k[0], v[0], [0, lq], [0, lk], True, 0.35)
    np.testing.assert_allclose(O, Of[0, lk - lq:], rtol=0, atol=1e-13)
    np.testing.assert_allclose(L, Lf[0][:, lk - lq:], rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_seqused_k_equals_truncated_keys(causal):
    rng = np.random.default_rng(7)
    qlens, klens, used = [3, 8], [20, 16], [12, 16]
    cu, q = _pack(qlens, 2, 8, rng)
    cuk, k = _pack(klens, 2, 8, rng)
    v = rng.standard_normal(k.shape)
    O, L = attention_varlen_ref(q, k, v, cu, cuk, causal, 0.3, seqused_k=used)
    for b in range(2):
        kk = k[cuk[b]:cuk[b] + used[b]]
        vv = v[cuk[b]:cuk[b] + used[b]]
        Ob, Lb = attention_varlen_ref(q[cu[b]:cu[b + 1]], kk, vv, [0, qlens[b]], [0, used[b]], causal, 0.3)
        np.testing.assert_allclose(O[cu[b]:cu[b + 1]], Ob, rtol=0, atol=1e-14)
        np.testing.assert_allclose(L[:, cu[b]:cu[b + 1]], Lb, rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_paged_cache_equals_packed_keys(causal):
    # build a packed K/V, scatter it into shuffled pages, and compare
    rng = np.random.default_rng(8)
    P, H, d = 4, 2, 8
    qlens, klens = [1, 5, 3], [9, 4, 13]
    cu, q = _pack(qlens, 4, d, rng)
    cuk, k = _pack(klens, H, d, rng)
    v = rng.standard_normal(k.shape)
    maxp = max((n + P - 1) // P for n in klens)
    npages = 3 * maxp + 2
    perm = rng.permutation(npages)
    kc = rng.standard_normal((npages, P, H, d))   # junk outside the used rows
    vc = rng.standard_normal((npages, P, H, d))
    bt = np.zeros((3, maxp), dtype=np.int64)
    nxt = 0
    for b, n in enumerate(klens):
        for lp in range((n + P - 1) // P):
            bt[b, lp] = perm[nxt]
            nxt += 1
        for t in range(n):
            kc[bt[b, t // P], t % P] = k[cuk[b] + t]
            vc[bt[b, t // P], t % P] = v[cuk[b] + t]
    O1, L1 = attention_paged_ref(q, kc, vc, cu, klens, bt, causal, 0.3)
    O2, L2 = attention_varlen_ref(q, k, v, cu, cuk, causal, 0.3)
    np.testing.assert_array_equal(O1, O2)
    np.testing.assert_array_equal(L1, L2)


def test_gqa_groups_are_contiguous():
    rng = np.random.default_rng(9)
    cu, q = _pack([6, 2], 4, 8, rng)
    _, k = _pack([6, 2], 2, 8, rng)
    v = rng.standard_normal(k.shape)
    O, L = attention_varlen_ref(q, k, v, cu, cu, True, 0.3)
    Or, Lr = attention_varlen_ref(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1), cu, cu, True, 0.3)
    np.testing.assert_array_equal(O, Or)
    np.testing.assert_array_equal(L, Lr)


# --- planted mutants must fail a pin

MUTANTS = {
    "top_left_alignment": ("(j <= i + (lk - lq))", "(j <= i)"),
    "mask_includes_next_key": ("(j <= i + (lk - lq))", "(j <= i + 1 + (lk - lq))"),
    "seqused_ignored": ("k1 = k0 + min(int(used[b]), k1 - k0)", "k1 = k1"),
    "page_row_and_page_swapped": ("pages, rows = bt[b, t // page_size], t % page_size",
                                  "pages, rows = bt[b, t % page_size], t // page_size"),
    "empty_rows_lse_zero": ("lse[h] = np.where(any_visible, m[:, 0] + np.log(safe[:, 0]), -np.inf)",
                            "lse[h] = np.where(any_visible, m[:, 0] + np.log(safe[:, 0]), 0.0)"),
    "gqa_modulo": ("kvh = h // group", "kvh = h % hkv"),
}


def _pins_pass(mod):
    tests = [
        test_bottom_right_two_queries_three_keys,
        test_more_queries_than_keys_leaves_empty_rows,
        test_decode_rows_see_every_key,
        test_chunked_prefill_equals_rows_of_the_full_causal_square,
        lambda: test_seqused_k_equals_truncated_keys(True),
        lambda: test_paged_cache_equals_packed_keys(True),
        test_gqa_groups_are_contiguous,
    ]
    g = globals()
    saved = (g["attention_varlen_ref"], g["attention_paged_ref"])
    g["attention_varlen_ref"], g["attention_paged_ref"] = mod.attention_varlen_ref, mod.attention_paged_ref
    try:
        for t in tests:
            t()
    except AssertionError:
        return False
    finally:
        g["attention_varlen_ref"], g["attention_paged_ref"] = saved
    return True


def test_unmutated_passes():
    assert _pins_pass(vmod)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    src = inspect.getsource(vmod)
    assert old in src, old
    mod = types.ModuleType("varlen_mutant")
    exec(compile(src.replace(old, new), "varlen_mutant", "exec"), mod.__dict__)
    assert not _pins_pass(mod), f"mutant {name} survived"
