"""CPU oracle for the exact-attention forward pass (test infrastructure only).

This module is the reference that the GPU path is checked against. It is test
infrastructure: only the tests, the smoke check and the CPU-baseline leg of the
benchmark may import it. The product path never calls it, and it shares no code,
tables or helpers with the HIP library.

What it computes (the plain definition, in float64):

  For every batch b and query head h, with KV head kvh = floor(h / (Hq / Hkv)):
    S = scale * Q[b,:,h,:] @ K[b,:,kvh,:]^T                    (Nq x Nk)
    causal: S[i, j] = -inf for j > i                            (query i sees keys 0..i)
    m_i   = max_j S[i, j]
    P     = exp(S - m)          l_i = sum_j P[i, j]
    O[b, i, h, :] = (P @ V[b,:,kvh,:])[i] / l_i
    LSE[b, h, i]  = m_i + ln(l_i)

Sources, as the pages state them:
  * "FlashAttention 4: Snellere, Geheugenefficiente Aandacht voor LLM's", sections
    "Inleiding" and "Veelgestelde vragen": attention multiplies queries by keys,
    normalises the result with a softmax and multiplies it by the values; the
    FlashAttention family reaches that same exact result tile by tile without
    materialising Q.K^T ("Waarom aandachtkernels ..." section).
  * "h3-blackwell-runtime/FLASH4.md", section "API": tensors are in the native
    [batch, sequence, heads, head_dim] layout.
  * "[RFC] FA4 - head_dim=256 & head_dim=512", section "Performance Snapshot":
    causal and non-causal variants.
  * Same Dutch page, compatibility section: grouped-query attention means several
    query heads share one key/value projection.

Readings where the pages are silent (each is listed in the design notes):
  * the causal mask is aligned top-left (key j visible to query i iff j <= i);
    all workloads have Nq == Nk, where top-left and bottom-right coincide;
  * the GQA head map is contiguous groups: kvh = h // (Hq // Hkv);
  * the scale is an explicit argument (1/sqrt(d) in every workload);
  * LSE is the natural-log log-sum-exp of the *scaled* scores over visible keys,
    laid out [B, Hq, Nq].

The backward pass (attention_bwd_ref) is the gradient of sum(O * dO) with respect to
q, k and v, written out from the same definition (the pages list a backward pass next to
the forward: "[RFC] FA4 - head_dim=256 & head_dim=512", Phase 1 and the backward tables
of "Performance Snapshot").

Pins: tests/test_oracle.py checks this module against hand-worked cases, closed
forms, invariants, a brute-force per-row formulation with math.fsum and torch's
own CPU scaled_dot_product_attention in float64; tests/test_oracle_bwd.py checks the
backward against torch autograd in float64, central finite differences and closed forms.
Nothing here is "parity unpinned".
"""

from __future__ import annotations

import math

import numpy as np

__all__ = ["attention_ref", "attention_bruteforce", "attention_bwd_ref", "kv_head_of"]


def kv_head_of(h: int, hq: int, hkv: int) -> int:
    """KV head shared by query head h: contiguous groups of Hq/Hkv query heads."""
    if hq % hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return h // (hq // hkv)


def _as_f64(x) -> np.ndarray:
    """Exact conversion to float64 (bf16/fp16 values are exact in fp32 and fp64)."""
    if hasattr(x, "detach"):  # a torch tensor: go through float32, which holds bf16/fp16 exactly
        x = x.detach().cpu().float().numpy()
    return np.asarray(x, dtype=np.float64)


def torch_index(a: np.ndarray):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a))


def _slice_f64(x, b, rows, h) -> np.ndarray:
    """x[b, rows, h, :] as float64 (exact for bf16/fp16/fp32 inputs)."""
    if hasattr(x, "detach"):  # torch tensor: slice first, then widen
        if isinstance(rows, np.ndarray):
            rows = torch_index(rows)
        return x[b, rows, h, :].detach().cpu().double().numpy()
    return np.asarray(x[b, rows, h, :], dtype=np.float64)


def attention_ref(q, k, v, causal: bool, scale: float, rows=None):
    """Exact attention forward in float64.

    q: [B, Nq, Hq, d]; k, v: [B, Nk, Hkv, d] (numpy arrays or CPU torch tensors).
    rows: None for every query row, or an integer array of query indices, either
      1-D (same rows for every (b, h)) or shaped [B, Hq, R] (rows per (b, h)).
    Returns (O, LSE) as float64 numpy arrays:
      rows is None: O [B, Nq, Hq, d], LSE [B, Hq, Nq]
      rows given:   O [B, Hq, R, d],  LSE [B, Hq, R]
    Inputs are widened to float64 one (b, head) slice at a time.
    """
    B, Nq, Hq, d = q.shape
    Bk, Nk, Hkv, dk = k.shape
    if Bk != B or dk != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError("q/k/v shapes do not agree")
    if causal and Nq != Nk:
        raise ValueError("causal attention is defined here for Nq == Nk only")
    scale = float(scale)

    if rows is None:
        O = np.empty((B, Nq, Hq, d), dtype=np.float64)
        LSE = np.empty((B, Hq, Nq), dtype=np.float64)
    else:
        rows = np.asarray(rows, dtype=np.int64)
        if rows.ndim == 1:
            rows = np.broadcast_to(rows, (B, Hq, rows.shape[0]))
        R = rows.shape[2]
        O = np.empty((B, Hq, R, d), dtype=np.float64)
        LSE = np.empty((B, Hq, R), dtype=np.float64)

    all_k = slice(None)
    for b in range(B):
        cached = None
        for h in range(Hq):
            kvh = kv_head_of(h, Hq, Hkv)
            if cached is None or cached[0] != kvh:
                cached = (kvh, _slice_f64(k, b, all_k, kvh), _slice_f64(v, b, all_k, kvh))
            _, Kh, Vh = cached  # [Nk, d] each
            qi = np.arange(Nq) if rows is None else rows[b, h]
            Qh = _slice_f64(q, b, all_k if rows is None else qi, h)  # [R, d]
            S = scale * (Qh @ Kh.T)  # [R, Nk]
            if causal:
                S[np.arange(Nk)[None, :] > qi[:, None]] = -np.inf
            m = S.max(axis=1, keepdims=True)
            P = np.exp(S - m)
            l = P.sum(axis=1, keepdims=True)
            Oh = (P @ Vh) / l
            lse = m[:, 0] + np.log(l[:, 0])
            if rows is None:
                O[b, :, h, :] = Oh
                LSE[b, h, :] = lse
            else:
                O[b, h] = Oh
                LSE[b, h] = lse
    return O, LSE


def attention_bruteforce(q, k, v, causal: bool, scale: float):
    """Second formulation for tiny inputs: pure-Python loops, one query row at a time.

    Each dot product and each sum is an exactly rounded math.fsum; the softmax is
    written as weights exp(s_j - max) over the visible keys. Same layouts and
    outputs as attention_ref with rows=None (returned as nested float64 arrays).
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    B, Nq, Hq, d = q.shape
    _, Nk, Hkv, _ = k.shape
    g = Hq // Hkv
    O = np.zeros((B, Nq, Hq, d))
    LSE = np.zeros((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            kvh = h // g
            for i in range(Nq):
                visible = range(i + 1) if causal else range(Nk)
                s = {}
                for j in visible:
                    s[j] = float(scale) * math.fsum(q[b, i, h, t] * k[b, j, kvh, t] for t in range(d))
                mx = max(s.values())
                w = {j: math.exp(s[j] - mx) for j in s}
                den = math.fsum(w.values())
                for t in range(d):
                    O[b, i, h, t] = math.fsum(w[j] * v[b, j, kvh, t] for j in s) / den
                LSE[b, h, i] = mx + math.log(den)
    return O, LSE


def attention_bwd_ref(q, k, v, dout, causal: bool, scale: float):
    """Exact attention backward in float64: gradients of sum(O * dout) w.r.t. q, k and v.

    With S = scale * Q K^T (causal: -inf above the diagonal), P = softmax(S) per row,
    O = P V:
        dV = P^T dO
        dP = dO V^T
        dS = P * (dP - D),  D_i = sum_j P_ij dP_ij  (= sum_d dO_id O_id)
        dQ = scale * dS K
        dK = scale * dS^T Q
    For grouped-query heads, dK and dV of a KV head sum the contributions of every query
    head of its group. Layouts as in attention_ref: q/dout/dq [B, Nq, Hq, d], k/v/dk/dv
    [B, Nk, Hkv, d]. Returns (dq, dk, dv) as float64 numpy arrays.
    """
    B, Nq, Hq, d = q.shape
    _, Nk, Hkv, _ = k.shape
    if causal and Nq != Nk:
        raise ValueError("causal attention is defined here for Nq == Nk only")
    scale = float(scale)
    dq = np.zeros((B, Nq, Hq, d))
    dk = np.zeros((B, Nk, Hkv, d))
    dv = np.zeros((B, Nk, Hkv, d))
    all_rows = slice(None)
    for b in range(B):
        for h in range(Hq):
            kvh = kv_head_of(h, Hq, Hkv)
            Qh = _slice_f64(q, b, all_rows, h)
            Kh = _slice_f64(k, b, all_rows, kvh)
            Vh = _slice_f64(v, b, all_rows, kvh)
            dOh = _slice_f64(dout, b, all_rows, h)
            S = scale * (Qh @ Kh.T)
            if causal:
                S[np.arange(Nk)[None, :] > np.arange(Nq)[:, None]] = -np.inf
            m = S.max(axis=1, keepdims=True)
            P = np.exp(S - m)
            P /= P.sum(axis=1, keepdims=True)
            dv[b, :, kvh, :] += P.T @ dOh
            dP = dOh @ Vh.T
            D = (P * dP).sum(axis=1, keepdims=True)
            dS = P * (dP - D)
            dq[b, :, h, :] = scale * (dS @ Kh)
            dk[b, :, kvh, :] += scale * (dS.T @ Qh)
    return dq, dk, dv
