"""GPU parity of the variable-length, seqused_k and paged-K/V forward pass (fa_fwd_varlen,
fa_fwd_paged and their fp16 forms, through the Python binding) against the fp64 oracle
in oracle/varlen.py, element by element on every row of every sequence.

Tolerance: the dense path's, O max-abs <= 1e-2 and mean-abs <= 1e-3, LSE max-abs <= 1e-3;
elements with |O_ref| >= 4, where half a bf16 ulp (1.56e-2) already exceeds 1e-2, are held to
half an ulp plus the same margin as in test_parity.py (rows that see one or two keys reach the
extremes of V); rows that see no key must come back as exactly O = 0 and LSE = -inf. Causal masks are
aligned bottom-right (query i of a sequence sees keys j <= i + Lk - Lq).
"""

import numpy as np
import pytest
import torch

import exact_attention_06_amd as fa
from exact_attention_06_amd import workloads as W
from oracle import attention_paged_ref, attention_varlen_ref

from parity_record import record

pytestmark = pytest.mark.gpu

O_MAX, O_MEAN, LSE_MAX = 1e-2, 1e-3, 1e-3
EXCESS = O_MAX - 2.0 ** -7


def _say(msg):
    print(msg, flush=True)


def _compare(name, o, lse, O_ref, L_ref):
    mant = 7 if o.dtype == torch.bfloat16 else 10
    o = o.float().cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    empty_ref = np.isneginf(L_ref)
    assert np.array_equal(np.isneginf(lse), empty_ref), f"{name}: rows without keys differ"
    assert np.isfinite(o).all(), f"{name}: non-finite O"
    eo = np.abs(o - O_ref)
    el = np.abs(lse[~empty_ref] - L_ref[~empty_ref]) if (~empty_ref).any() else np.zeros(1)
    mx, mean, lmx = float(eo.max()), float(eo.mean()), float(el.max())
    big = np.abs(O_ref) >= 4.0
    half_ulp = 0.5 * np.exp2(np.floor(np.log2(np.maximum(np.abs(O_ref), 2.0 ** -126))) - mant)
    mx_small = float(eo[~big].max()) if (~big).any() else 0.0
    ex_big = float((eo - half_ulp)[big].max()) if big.any() else 0.0
    n_empty = int(empty_ref.sum())
    at = np.unravel_index(int(np.argmax(eo)), eo.shape)
    _say(f"  {name}: O max {mx:.3e} (|O_ref| there {abs(O_ref[at]):.3f}) mean {mean:.3e} | LSE max {lmx:.3e} | "
         f"|O_ref|>=4: {int(big.sum())} elems, excess {ex_big:.3e} | empty rows (x heads) {n_empty}")
    record(case=name, o_max=mx, o_max_small=mx_small, o_mean=mean, lse_max=lmx, n_big=int(big.sum()), ex_big=ex_big)
    if n_empty:
        rows_empty = empty_ref.any(axis=0)
        assert np.all(o[rows_empty] == 0.0), f"{name}: empty rows must be exactly 0"
    assert mx_small <= O_MAX and ex_big <= EXCESS and mean <= O_MEAN and lmx <= LSE_MAX, \
        f"{name}: O max {mx:.3e} (|O|<4 {mx_small:.3e}, excess {ex_big:.3e}) mean {mean:.3e} LSE max {lmx:.3e}"


def _run_varlen(name, Lq, Lk, Hq, Hkv, d, causal, seed, used=None, dtype=torch.bfloat16, splits=0, scale=None):
    q, k, v, cu_q, cu_k = W.make_varlen(Lq, Lk, Hq, Hkv, d, seed, dtype)
    if scale is None:
        scale = float(torch.tensor(d ** -0.5, dtype=torch.float32))
    _say(f"[gpu] varlen {name} B={len(Lq)} Lq={list(Lq)[:8]} Lk={list(Lk)[:8]} used={used} Hq={Hq} "
         f"Hkv={Hkv} d={d} causal={causal} {dtype} splits={splits}")
    used_t = None if used is None else torch.tensor(used, dtype=torch.int32)
    o, lse = fa.forward_varlen(q.cuda(), k.cuda(), v.cuda(), cu_q.cuda(), cu_k.cuda(), max(Lq), causal=causal,
                               scale=scale, seqused_k=None if used_t is None else used_t.cuda(), num_splits=splits)
    torch.cuda.synchronize()
    O_ref, L_ref = attention_varlen_ref(q, k, v, cu_q, cu_k, causal, scale, seqused_k=used_t)
    _compare(name, o, lse, O_ref, L_ref)


def _run_paged(name, Lq, used, page_size, Hq, Hkv, d, causal, seed, dtype=torch.bfloat16, splits=0, scale=None):
    q, kc, vc, cu_q, used_t, bt = W.make_paged(Lq, used, page_size, Hq, Hkv, d, seed, dtype)
    if scale is None:
        scale = float(torch.tensor(d ** -0.5, dtype=torch.float32))
    _say(f"[gpu] paged {name} B={len(Lq)} Lq={list(Lq)[:8]} used={list(used)[:8]} page={page_size} "
         f"pages={kc.shape[0]} Hq={Hq} Hkv={Hkv} d={d} causal={causal} {dtype} splits={splits}")
    o, lse = fa.forward_paged(q.cuda(), kc.cuda(), vc.cuda(), cu_q.cuda(), used_t.cuda(), bt.cuda(), max(Lq),
                              causal=causal, scale=scale, num_splits=splits)
    torch.cuda.synchronize()
    O_ref, L_ref = attention_paged_ref(q, kc, vc, cu_q, used_t, bt, causal, scale)
    _compare(name, o, lse, O_ref, L_ref)


VARLEN = [
    # name,            Lq,                          Lk,                          Hq, Hkv, d,  seed, used
    ("equal_lengths",  (1, 63, 64, 65, 200, 513),   (1, 63, 64, 65, 200, 513),   4, 2, 128, 41, None),
    ("equal_hd256",    (1, 31, 32, 33, 129, 300),   (1, 31, 32, 33, 129, 300),   2, 1, 256, 42, None),
    ("q_shorter",      (5, 100, 300, 64),           (300, 700, 300, 65),         4, 2, 128, 43, None),
    ("q_shorter_256",  (5, 100, 300),               (300, 700, 301),             2, 2, 256, 44, None),
    ("q_longer",       (100, 257, 40),              (30, 1, 40),                 4, 1, 128, 45, None),
    ("q_longer_256",   (100, 140),                  (30, 3),                     2, 1, 256, 46, None),
    ("decode",         (1,) * 8,                    (1, 5, 64, 65, 129, 1000, 2047, 3000), 4, 4, 128, 47, None),
    ("seqused",        (40, 100, 300, 77),          (64, 100, 300, 90),          4, 2, 128, 48, (0, 17, 300, 90)),
    ("seqused_256",    (40, 100, 300),              (64, 100, 300),              2, 2, 256, 49, (0, 33, 250)),
]


@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
@pytest.mark.parametrize("case", VARLEN, ids=[c[0] for c in VARLEN])
def test_varlen(case, causal):
    name, Lq, Lk, Hq, Hkv, d, seed, used = case
    _run_varlen(name, Lq, Lk, Hq, Hkv, d, causal, seed, used)


PAGED = [
    # name,            Lq,                 seqused_k,                   page, Hq, Hkv, d, seed
    ("pages64_hd128",  (1, 7, 64, 130),    (64, 1000, 64, 500),         64,  4, 2, 128, 51),
    ("pages128_hd128", (1, 16, 300, 2),    (0, 129, 1500, 2048),        128, 4, 1, 128, 52),
    ("pages64_hd256",  (3, 33, 100),       (100, 33, 1000),             64,  2, 2, 256, 53),
    ("pages128_hd256", (1, 1, 12, 256),    (1, 4000, 127, 256),         128, 2, 1, 256, 54),
]


@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
@pytest.mark.parametrize("case", PAGED, ids=[c[0] for c in PAGED])
def test_paged(case, causal):
    name, Lq, used, page, Hq, Hkv, d, seed = case
    _run_paged(name, Lq, used, page, Hq, Hkv, d, causal, seed)


@pytest.mark.parametrize("d", [128, 256])
def test_fp16_entry_points(d):
    _run_varlen(f"fp16_varlen_d{d}", (17, 200), (300, 200), 2, 1, d, True, 55 + d, dtype=torch.float16)
    _run_paged(f"fp16_paged_d{d}", (3, 64), (700, 64), 128, 2, 1, d, True, 56 + d, dtype=torch.float16)


@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
@pytest.mark.parametrize("d", [128, 256])
def test_negative_scale(d, causal):
    # scale -1/sqrt(d): scores of the opposite sign, packed and paged, without and with splits
    sc = -float(d) ** -0.5
    _run_varlen(f"neg_varlen_d{d}", (17, 200, 64), (300, 200, 64), 4, 2, d, causal, 57 + d, scale=sc)
    _run_paged(f"neg_paged_d{d}", (3, 64), (700, 64), 128, 2, 1, d, causal, 58 + d, scale=sc)
    _run_paged(f"neg_paged_split_d{d}", (1, 4), (900, 3000), 128, 2, 1, d, causal, 59 + d, scale=sc, splits=4)


def test_paged_equals_varlen_on_the_same_keys():
    # the same logical keys, packed or scattered over shuffled pages, give bitwise equal O
    d, Hq, Hkv, page = 128, 4, 2, 128
    Lq, Lk = (9, 200), (1000, 300)
    q, kc, vc, cu_q, used, bt = W.make_paged(Lq, Lk, page, Hq, Hkv, d, 57)
    k = torch.cat([kc[bt[b, t // page], t % page][None] for b in range(2) for t in range(Lk[b])])
    v = torch.cat([vc[bt[b, t // page], t % page][None] for b in range(2) for t in range(Lk[b])])
    cu_k = torch.tensor([0, Lk[0], Lk[0] + Lk[1]], dtype=torch.int32)
    o1, l1 = fa.forward_paged(q.cuda(), kc.cuda(), vc.cuda(), cu_q.cuda(), used.cuda(), bt.cuda(), max(Lq),
                              causal=True)
    o2, l2 = fa.forward_varlen(q.cuda(), k.cuda(), v.cuda(), cu_q.cuda(), cu_k.cuda(), max(Lq), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_varlen_equals_dense_for_one_square_sequence():
    # one sequence with Lq == Lk: the variable-length kernel matches the dense one bitwise
    for d in (128, 256):
        q, k, v, cu_q, cu_k = W.make_varlen((777,), (777,), 4, 2, d, 58)
        for causal in (False, True):
            o1, l1 = fa.forward_varlen(q.cuda(), k.cuda(), v.cuda(), cu_q.cuda(), cu_k.cuda(), 777, causal=causal)
            o2, l2 = fa.forward(q[None].cuda(), k[None].cuda(), v[None].cuda(), causal=causal)
            torch.cuda.synchronize()
            assert torch.equal(o1, o2[0]) and torch.equal(l1, l2[0]), (d, causal)


VW = W.var_workloads()


@pytest.mark.parametrize("w", VW, ids=[w.name for w in VW])
def test_var_workloads(w):
    for causal in w.causal_modes:
        if w.paged:
            _run_paged(w.name, w.seqlens_q, w.seqlens_k, w.page_size, w.Hq, w.Hkv, w.d, causal, w.seed)
        else:
            _run_varlen(w.name, w.seqlens_q, w.seqlens_k, w.Hq, w.Hkv, w.d, causal, w.seed)


# ---------------------------------------------------------------- seeded random batches

def _random_varlen(i):
    g = np.random.default_rng(3000 + i)
    B = int(g.integers(1, 7))
    Lq = [int(x) for x in g.integers(0, 400, B)]
    if sum(Lq) == 0:
        Lq[0] = 1
    causal = bool(g.integers(0, 2))
    Lk = [int(x) for x in g.integers(0, 900, B)]
    used = [int(g.integers(0, n + 1)) for n in Lk] if g.integers(0, 2) else None
    hkv = int(g.choice([1, 2, 4]))
    return (f"rv{i}", tuple(Lq), tuple(Lk), hkv * int(g.choice([1, 2])), hkv, int(g.choice([128, 256])), causal,
            4000 + i, None if used is None else tuple(used))


def _random_paged(i):
    g = np.random.default_rng(5000 + i)
    B = int(g.integers(1, 7))
    Lq = tuple(int(x) for x in g.integers(1, 200, B))
    used = tuple(int(x) for x in g.integers(0, 1500, B))
    hkv = int(g.choice([1, 2, 4]))
    return (f"rp{i}", Lq, used, int(g.choice([64, 128, 192, 256])), hkv * int(g.choice([1, 2])), hkv,
            int(g.choice([128, 256])), bool(g.integers(0, 2)), 6000 + i)


RV = [_random_varlen(i) for i in range(12)]
RP = [_random_paged(i) for i in range(12)]


@pytest.mark.parametrize("case", RV, ids=[c[0] for c in RV])
def test_random_varlen(case):
    name, Lq, Lk, Hq, Hkv, d, causal, seed, used = case
    _run_varlen(name, Lq, Lk, Hq, Hkv, d, causal, seed, used)


@pytest.mark.parametrize("case", RP, ids=[c[0] for c in RP])
def test_random_paged(case):
    name, Lq, used, page, Hq, Hkv, d, causal, seed = case
    _run_paged(name, Lq, used, page, Hq, Hkv, d, causal, seed)



# ---------------------------------------------------------------- split-KV forms

@pytest.mark.parametrize("splits", [2, 3, 8])
@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
@pytest.mark.parametrize("case", VARLEN, ids=[c[0] for c in VARLEN])
def test_varlen_splitkv(case, causal, splits):
    name, Lq, Lk, Hq, Hkv, d, seed, used = case
    _run_varlen(f"{name}/s{splits}", Lq, Lk, Hq, Hkv, d, causal, seed, used, splits=splits)


@pytest.mark.parametrize("splits", [2, 5])
@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
@pytest.mark.parametrize("case", PAGED, ids=[c[0] for c in PAGED])
def test_paged_splitkv(case, causal, splits):
    name, Lq, used, page, Hq, Hkv, d, seed = case
    _run_paged(f"{name}/s{splits}", Lq, used, page, Hq, Hkv, d, causal, seed, splits=splits)


@pytest.mark.parametrize("case", RV, ids=[c[0] for c in RV])
def test_random_varlen_splitkv(case):
    name, Lq, Lk, Hq, Hkv, d, causal, seed, used = case
    _run_varlen(name + "/split", Lq, Lk, Hq, Hkv, d, causal, seed, used, splits=1 + seed % 7)


@pytest.mark.parametrize("case", RP, ids=[c[0] for c in RP])
def test_random_paged_splitkv(case):
    name, Lq, used, page, Hq, Hkv, d, causal, seed = case
    _run_paged(name + "/split", Lq, used, page, Hq, Hkv, d, causal, seed, splits=1 + seed % 9)


@pytest.mark.parametrize("d", [128, 256])
def test_fp16_splitkv(d):
    _run_varlen(f"fp16_varlen_split_d{d}", (17, 200), (300, 200), 2, 1, d, True, 65 + d, dtype=torch.float16,
                splits=3)
    _run_paged(f"fp16_paged_split_d{d}", (3, 64), (700, 64), 128, 2, 1, d, True, 66 + d, dtype=torch.float16,
               splits=4)


@pytest.mark.parametrize("d", [128, 256])
def test_one_split_equals_no_split_bitwise(d):
    # one split: each block covers all keys, the merge has one weight of exactly 1
    q, kc, vc, cu_q, used, bt = W.make_paged((1, 9, 200), (700, 1000, 300), 128, 4, 2, d, 67)
    for causal in (False, True):
        o1, l1 = fa.forward_paged(q.cuda(), kc.cuda(), vc.cuda(), cu_q.cuda(), used.cuda(), bt.cuda(), 200,
                                  causal=causal)
        o2, l2 = fa.forward_paged(q.cuda(), kc.cuda(), vc.cuda(), cu_q.cuda(), used.cuda(), bt.cuda(), 200,
                                  causal=causal, num_splits=1)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), (d, causal)


def test_decode_workload_splitkv():
    w = [x for x in W.var_workloads() if x.paged and "decode" in x.name][0]
    for splits in (4, 16):
        _run_paged(f"{w.name}/s{splits}", w.seqlens_q, w.seqlens_k, w.page_size, w.Hq, w.Hkv, w.d, True, w.seed,
                   splits=splits)


# Batches of at most 64 sequences are dispatched sequence by sequence, longest first (each block
# ranks the sequences by key count across a wave; causal: a sequence's highest query tile
# first); more than 64 take the other order. Cover the limit, one past it, tied key counts,
# empty sequences, rows that see no key (causal, more queries than keys) and a head count that
# is not a multiple of 8 (the head order inside an entry differs then).
def _lpt_lengths(n, seed):
    g = np.random.default_rng(seed)
    Lq = [int(x) for x in g.integers(0, 300, n)]
    Lk = [int(x) for x in g.choice([0, 64, 64, 130, 257, 700], n)]  # many ties, some empty
    return tuple(Lq), tuple(Lk)


@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
@pytest.mark.parametrize("n,Hq,Hkv,d", [(64, 8, 2, 128), (65, 8, 2, 128), (64, 6, 3, 256), (40, 16, 4, 128),
                                        (1, 8, 8, 256)])
def test_varlen_longest_first_order(n, Hq, Hkv, d, causal):
    Lq, Lk = _lpt_lengths(n, 500 + n + d)
    _run_varlen(f"lpt{n}_h{Hq}_d{d}", Lq, Lk, Hq, Hkv, d, causal, 600 + n)


@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
@pytest.mark.parametrize("n", [64, 65])
def test_paged_longest_first_order(n, causal):
    g = np.random.default_rng(700 + n)
    Lq = tuple(int(x) for x in g.integers(1, 200, n))
    used = tuple(int(x) for x in g.choice([0, 128, 128, 300, 640], n))
    _run_paged(f"lpt_paged{n}", Lq, used, 128, 8, 8, 256, causal, 800 + n)
