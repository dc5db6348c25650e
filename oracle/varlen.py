"""CPU oracle for variable-length, key-length-limited and paged-K/V attention (test
infrastructure only: imported by the tests, never by the library or its binding).

These are the serving variants that the pages list next to the dense forward pass: packed
variable-length batches, per-sequence used key counts ("seqused_k") and a paged K/V cache
whose page size equals the key tile ("[RFC] FA4 - head_dim=256 & head_dim=512", the
feature table of section "Phase 2"; the Dutch page, section "Compatibiliteit en huidige
status", for varlen). What each sequence computes is the plain definition of the dense
oracle, applied to that sequence alone, in float64:

  For sequence b with Lq query rows and Lk keys, query head h and KV head
  kvh = h // (Hq / Hkv):
    S = scale * Q_b[:, h, :] @ K_b[:, kvh, :]^T                 (Lq x Lk)
    causal: query i sees key j iff j <= i + (Lk - Lq)           (bottom-right alignment)
    O_b[i, h, :] = softmax(S[i, visible]) @ V_b[visible, kvh, :]
    LSE[h, q0 + i] = log-sum-exp of S[i, visible]
  A row that sees no key (Lk = 0, or i + Lk - Lq < 0 under the causal mask) has O = 0 and
  LSE = -inf.

Readings where the pages are silent (each is listed in the design notes):
  * causal alignment for Lq != Lk is bottom-right: the last query row sees every key, as
    in decoding against a cache; for Lq == Lk it is the dense path's top-left mask;
  * packed layouts: q and o are [total_q, Hq, d], packed k and v are [total_k, Hkv, d],
    LSE is [Hq, total_q]; sequence b owns rows cu_seqlens[b] .. cu_seqlens[b+1]-1;
  * seqused_k[b] keys of sequence b are used (the first ones); further rows are ignored;
  * paged: k_cache and v_cache are [num_pages, page_size, Hkv, d]; logical key t of
    sequence b lives in page block_table[b, t // page_size], row t % page_size.

Pins: tests/test_oracle_varlen.py (hand-worked bottom-right cases, decode rows against the
non-causal dense oracle, equal-length sequences against the dense oracle, empty rows,
seqused_k against truncated keys, paged against packed with shuffled pages).
"""

from __future__ import annotations

import numpy as np

__all__ = ["attention_varlen_ref", "attention_paged_ref", "gather_paged"]


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu().float().numpy()
    return np.asarray(x, dtype=np.float64)


def _ints(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.asarray(x, dtype=np.int64)


def _one_sequence(qb, kb, vb, causal, scale, hq, hkv):
    """qb [Lq, Hq, d], kb/vb [Lk, Hkv, d] in float64 -> O [Lq, Hq, d], LSE [Hq, Lq]."""
    lq, lk = qb.shape[0], kb.shape[0]
    d = qb.shape[2]
    o = np.zeros((lq, hq, d))
    lse = np.full((hq, lq), -np.inf)
    if lq == 0 or lk == 0:
        return o, lse
    group = hq // hkv
    i = np.arange(lq)[:, None]
    j = np.arange(lk)[None, :]
    visible = (j <= i + (lk - lq)) if causal else np.ones((lq, lk), dtype=bool)
    any_visible = visible.any(axis=1)
    for h in range(hq):
        kvh = h // group
        s = scale * (qb[:, h, :] @ kb[:, kvh, :].T)
        s = np.where(visible, s, -np.inf)
        m = np.max(s, axis=1, keepdims=True)
        m = np.where(any_visible[:, None], m, 0.0)
        p = np.exp(s - m)                          # exp(-inf) = 0 for masked keys
        l = p.sum(axis=1, keepdims=True)
        safe = np.where(l > 0, l, 1.0)
        o[:, h, :] = np.where(any_visible[:, None], (p @ vb[:, kvh, :]) / safe, 0.0)
        lse[h] = np.where(any_visible, m[:, 0] + np.log(safe[:, 0]), -np.inf)
    return o, lse


def attention_varlen_ref(q, k, v, cu_seqlens_q, cu_seqlens_k, causal: bool, scale: float,
                         seqused_k=None):
    """Packed variable-length attention in float64.

    q: [total_q, Hq, d]; k, v: [total_k, Hkv, d]; cu_seqlens_q, cu_seqlens_k: B+1 offsets;
    seqused_k: None or B key counts (at most cu_seqlens_k[b+1] - cu_seqlens_k[b]).
    Returns O [total_q, Hq, d] and LSE [Hq, total_q] (float64 numpy).
    """
    qf, kf, vf = _f64(q), _f64(k), _f64(v)
    cq, ck = _ints(cu_seqlens_q), _ints(cu_seqlens_k)
    used = None if seqused_k is None else _ints(seqused_k)
    total_q, hq, d = qf.shape
    hkv = kf.shape[1]
    if hq % hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    o = np.zeros((total_q, hq, d))
    lse = np.full((hq, total_q), -np.inf)
    for b in range(len(cq) - 1):
        q0, q1 = int(cq[b]), int(cq[b + 1])
        k0, k1 = int(ck[b]), int(ck[b + 1])
        if used is not None:
            k1 = k0 + min(int(used[b]), k1 - k0)
        ob, lb = _one_sequence(qf[q0:q1], kf[k0:k1], vf[k0:k1], causal, scale, hq, hkv)
        o[q0:q1] = ob
        lse[:, q0:q1] = lb
    return o, lse


def gather_paged(cache, block_table, b: int, length: int) -> np.ndarray:
    """Logical rows 0..length-1 of sequence b from a paged cache [pages, page_size, H, d]."""
    bt = _ints(block_table)
    page_size = cache.shape[1]
    t = np.arange(length)
    pages, rows = bt[b, t // page_size], t % page_size
    if hasattr(cache, "detach"):  # torch tensor: gather first, then widen (exact)
        import torch
        return _f64(cache[torch.from_numpy(pages), torch.from_numpy(rows)])
    c = np.asarray(cache)
    return np.asarray(c[pages, rows], dtype=np.float64)


def attention_paged_ref(q, k_cache, v_cache, cu_seqlens_q, seqused_k, block_table, causal: bool,
                        scale: float):
    """Attention against a paged K/V cache in float64.

    q: [total_q, Hq, d]; k_cache, v_cache: [num_pages, page_size, Hkv, d];
    seqused_k: B key counts; block_table: [B, max_pages] physical page of each logical page.
    Returns O [total_q, Hq, d] and LSE [Hq, total_q] (float64 numpy).
    """
    qf = _f64(q)
    cq, used = _ints(cu_seqlens_q), _ints(seqused_k)
    total_q, hq, d = qf.shape
    hkv = k_cache.shape[2]
    if hq % hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    o = np.zeros((total_q, hq, d))
    lse = np.full((hq, total_q), -np.inf)
    for b in range(len(cq) - 1):
        q0, q1 = int(cq[b]), int(cq[b + 1])
        kb = gather_paged(k_cache, block_table, b, int(used[b]))
        vb = gather_paged(v_cache, block_table, b, int(used[b]))
        ob, lb = _one_sequence(qf[q0:q1], kb, vb, causal, scale, hq, hkv)
        o[q0:q1] = ob
        lse[:, q0:q1] = lb
    return o, lse
