"""Seeded synthetic inputs for the attention forward pass.

This module only draws numbers and names shapes; it holds none of the attention
arithmetic, so both the GPU path's tests and the CPU oracle can consume what it
produces. Inputs are drawn with torch's CPU generator (fp32 normal draws in the
order q, k, v) and rounded to the element dtype (round-to-nearest-even), so the
oracle and the kernel see the very same bf16/fp16 values.

Workload shapes follow the pages:
  * "h3-blackwell-runtime/FLASH4.md", "GB10 Validation" table: [1, 257, 8, 128]
    and [1, 20480, 56, 128] in [batch, seq, heads, head_dim];
  * "[RFC] FA4 - head_dim=256 & head_dim=512", "Performance Snapshot": head_dim 256,
    8 query heads, batch sized to about 32k tokens, sequence lengths 1k..128k; the same
    shape at head_dim 512, which the page's "Phase 4" table lists without shapes.
The head_dim=128 sweep (16 query heads, MHA and 4:1 GQA) and the spiked-key video
shape (every 16th key scaled by 4, to make peaked softmax rows) are synthetic
stand-ins with the same structure; there is no dataset behind any of them.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import torch

__all__ = ["Workload", "make_qkv", "sample_rows", "tiny", "ragged", "hd128_sweep",
           "hd256_sweep", "hd512_sweep", "video", "all_workloads", "by_name", "VarWorkload", "make_varlen",
           "make_paged", "var_workloads", "var_inputs"]

TOKENS = 32768  # batch is sized so that B * N is about this many tokens


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    N: int          # Nq == Nk
    Hq: int
    Hkv: int
    d: int
    seed: int
    causal_modes: tuple = (False, True)
    k_spike: bool = False          # scale every 16th key token by 4 (after rounding)
    full_oracle: bool = True       # oracle over all rows (else sampled rows)
    tags: tuple = field(default_factory=tuple)

    @property
    def scale(self) -> float:
        """1/sqrt(d), rounded to fp32 (the value the kernel receives)."""
        return float(torch.tensor(1.0 / self.d ** 0.5, dtype=torch.float32))

    def flops(self, causal: bool) -> float:
        """4*B*Hq*Nq*Nk*d, halved for causal (the reporting convention)."""
        f = 4.0 * self.B * self.Hq * self.N * self.N * self.d
        return f / 2 if causal else f


def make_qkv(B, Nq, Nk, Hq, Hkv, d, seed, dtype=torch.bfloat16, k_spike=False):
    """q [B,Nq,Hq,d], k and v [B,Nk,Hkv,d]: i.i.d. N(0,1) fp32 draws, rounded to dtype.

    With k_spike, key tokens j with j % 16 == 0 (all heads) are multiplied by 4
    after rounding; the product is exact in bf16/fp16.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    q = torch.randn((B, Nq, Hq, d), generator=g, dtype=torch.float32).to(dtype)
    k = torch.randn((B, Nk, Hkv, d), generator=g, dtype=torch.float32).to(dtype)
    v = torch.randn((B, Nk, Hkv, d), generator=g, dtype=torch.float32).to(dtype)
    if k_spike:
        k[:, 0::16] *= 4
    return q, k, v


def sample_rows(B, Hq, Nq, seed, R=64):
    """Query rows checked per (b, h) when the full oracle would be too slow.

    Always includes the first rows, tile and wave boundaries and the last rows;
    the rest are drawn with torch.randint from seed + 100. Returns int64 [B, Hq, R].
    """
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, 255, 256, Nq // 2, Nq - 2, Nq - 1]
    fixed = sorted({r for r in fixed if 0 <= r < Nq})
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed) + 100)
    rnd = torch.randint(0, Nq, (B, Hq, max(0, R - len(fixed))), generator=g)
    fx = torch.tensor(fixed, dtype=torch.int64).expand(B, Hq, len(fixed))
    return torch.cat([fx, rnd], dim=2)[:, :, :R].contiguous()


def tiny():
    return Workload("tiny", B=1, N=256, Hq=2, Hkv=2, d=128, seed=1)


def ragged():
    return Workload("ragged", B=1, N=257, Hq=8, Hkv=8, d=128, seed=2)


def hd128_sweep():
    out = []
    for i, N in enumerate([1024, 2048, 4096, 8192, 16384, 32768]):
        for hkv in (16, 4):
            out.append(Workload(f"hd128_N{N}_{'mha' if hkv == 16 else 'gqa4'}", B=TOKENS // N, N=N,
                                Hq=16, Hkv=hkv, d=128, seed=3 + i, full_oracle=N <= 4096))
    return out


def hd256_sweep():
    out = []
    for i, N in enumerate([1024, 2048, 4096, 8192, 16384, 32768, 65536, 131072]):
        out.append(Workload(f"hd256_N{N}", B=max(1, TOKENS // N), N=N, Hq=8, Hkv=8, d=256,
                            seed=4 + i, full_oracle=False))
    return out


def hd512_sweep():
    """Head dim 512 (the pages list it as a planned extended head dim, with no shapes of its
    own): the hd256 snapshot's shape - 8 query heads, about 32k tokens - at d = 512."""
    out = []
    for i, N in enumerate([1024, 2048, 4096, 8192, 16384, 32768]):
        out.append(Workload(f"hd512_N{N}", B=max(1, TOKENS // N), N=N, Hq=8, Hkv=8, d=512,
                            seed=60 + i, full_oracle=False))
    return out


def video():
    return Workload("video", B=1, N=20480, Hq=56, Hkv=56, d=128, seed=5, causal_modes=(False,),
                    k_spike=True, full_oracle=False)


def all_workloads():
    return [tiny(), ragged()] + hd128_sweep() + hd256_sweep() + [video()] + hd512_sweep()


def by_name(name):
    for w in all_workloads():
        if w.name == name:
            return w
    raise KeyError(name)


def inputs_for(w: Workload, dtype=torch.bfloat16):
    return make_qkv(w.B, w.N, w.N, w.Hq, w.Hkv, w.d, w.seed, dtype=dtype, k_spike=w.k_spike)


# ---- variable-length batches and paged K/V caches (the serving variants: "[RFC] FA4 -
#      head_dim=256 & head_dim=512", feature table of section "Phase 2"). Sequence lengths,
#      page orders and values are seeded draws; nothing here computes attention.

@dataclass(frozen=True)
class VarWorkload:
    name: str
    seqlens_q: tuple       # query rows per sequence
    seqlens_k: tuple       # keys per sequence (paged: seqused_k)
    Hq: int
    Hkv: int
    d: int
    seed: int
    paged: bool = False
    page_size: int = 128
    causal_modes: tuple = (False, True)

    @property
    def B(self) -> int:
        return len(self.seqlens_q)

    @property
    def scale(self) -> float:
        return float(torch.tensor(1.0 / self.d ** 0.5, dtype=torch.float32))

    def flops(self, causal: bool) -> float:
        """4*Hq*d per visible (query, key) pair; causal is aligned bottom-right."""
        pairs = 0
        for lq, lk in zip(self.seqlens_q, self.seqlens_k):
            if not causal:
                pairs += lq * lk
            else:
                # row i sees min(lk, max(0, i + 1 + lk - lq)) keys
                for i in range(lq):
                    pairs += min(lk, max(0, i + 1 + lk - lq))
        return 4.0 * self.Hq * self.d * pairs


def _lengths(n, lo, hi, seed):
    """n lengths drawn log-uniformly in [lo, hi] (seeded)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    u = torch.rand(n, generator=g, dtype=torch.float64)
    return tuple(int(x) for x in torch.exp(torch.log(torch.tensor(float(lo))) +
                                            u * (torch.log(torch.tensor(float(hi))) -
                                                 torch.log(torch.tensor(float(lo))))).round())


def make_varlen(seqlens_q, seqlens_k, Hq, Hkv, d, seed, dtype=torch.bfloat16, device="cpu"):
    """Packed q [sum Lq, Hq, d], k and v [sum Lk, Hkv, d] (N(0,1) draws rounded to dtype)
    and int32 offsets cu_seqlens_q, cu_seqlens_k (CPU tensors). device="cuda" draws the
    values on the GPU (other numbers, same distribution: for timing only)."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    tq, tk = int(sum(seqlens_q)), int(sum(seqlens_k))
    q = torch.randn((tq, Hq, d), generator=g, dtype=torch.float32, device=device).to(dtype)
    k = torch.randn((tk, Hkv, d), generator=g, dtype=torch.float32, device=device).to(dtype)
    v = torch.randn((tk, Hkv, d), generator=g, dtype=torch.float32, device=device).to(dtype)
    cu_q = torch.tensor([0] + list(torch.cumsum(torch.tensor(seqlens_q), 0).tolist()), dtype=torch.int32)
    cu_k = torch.tensor([0] + list(torch.cumsum(torch.tensor(seqlens_k), 0).tolist()), dtype=torch.int32)
    return q, k, v, cu_q, cu_k


def make_paged(seqlens_q, seqused_k, page_size, Hq, Hkv, d, seed, dtype=torch.bfloat16, spare_pages=3,
               device="cpu"):
    """Packed q [sum Lq, Hq, d]; k_cache, v_cache [num_pages, page_size, Hkv, d] filled with
    N(0,1) draws everywhere (rows past a sequence's keys hold unrelated values); a
    block_table [B, max_pages] int32 that hands out the pages in a seeded random order
    (unused entries point at page 0); int32 cu_seqlens_q and seqused_k. CPU tensors
    (device="cuda": q and the caches are drawn on the GPU, for timing only)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    gv = g if device == "cpu" else torch.Generator(device=device)
    if device != "cpu":
        gv.manual_seed(int(seed))
    B = len(seqlens_q)
    need = [(n + page_size - 1) // page_size for n in seqused_k]
    max_pages = max(1, max(need))
    num_pages = sum(need) + spare_pages
    q = torch.randn((int(sum(seqlens_q)), Hq, d), generator=gv, dtype=torch.float32, device=device).to(dtype)
    kc = torch.randn((num_pages, page_size, Hkv, d), generator=gv, dtype=torch.float32, device=device).to(dtype)
    vc = torch.randn((num_pages, page_size, Hkv, d), generator=gv, dtype=torch.float32, device=device).to(dtype)
    perm = torch.randperm(num_pages, generator=g)
    bt = torch.zeros((B, max_pages), dtype=torch.int32)
    nxt = 0
    for b in range(B):
        for p in range(need[b]):
            bt[b, p] = int(perm[nxt])
            nxt += 1
    cu_q = torch.tensor([0] + list(torch.cumsum(torch.tensor(seqlens_q), 0).tolist()), dtype=torch.int32)
    used = torch.tensor(list(seqused_k), dtype=torch.int32)
    return q, kc, vc, cu_q, used, bt


def varlen_prefill():
    """Packed prefill batch: 12 sequences of 64..4096 tokens (log-uniform), Lq == Lk,
    hd128, 16 query heads over 4 KV heads."""
    L = _lengths(12, 64, 4096, 31)
    return VarWorkload("varlen_prefill_hd128", L, L, 16, 4, 128, 31)


def chunked_prefill():
    """Chunked prefill against a cache: 8 sequences, 512 new query rows each against
    1024..8192 keys (bottom-right causal), hd128, 16 over 4 heads."""
    Lk = _lengths(8, 1024, 8192, 32)
    return VarWorkload("chunked_prefill_hd128", (512,) * 8, Lk, 16, 4, 128, 32, causal_modes=(True,))


def paged_decode():
    """Paged decode: 32 sequences with 1..16 new query rows (speculative decoding) against
    256..16384 cached keys in 128-key pages, hd256, 8 query heads over 8 KV heads."""
    Lk = _lengths(32, 256, 16384, 33)
    g = torch.Generator(device="cpu")
    g.manual_seed(34)
    Lq = tuple(int(x) for x in torch.randint(1, 17, (32,), generator=g))
    return VarWorkload("paged_decode_hd256", Lq, Lk, 8, 8, 256, 33, paged=True, page_size=128,
                       causal_modes=(True,))


def paged_prefill():
    """Paged prefill: 6 sequences of 128..4096 tokens (Lq == Lk) in 128-key pages, hd256,
    8 query heads over 8 KV heads."""
    L = _lengths(6, 128, 4096, 35)
    return VarWorkload("paged_prefill_hd256", L, L, 8, 8, 256, 35, paged=True, page_size=128)


def var_workloads():
    return [varlen_prefill(), chunked_prefill(), paged_decode(), paged_prefill()]


def var_inputs(w: VarWorkload, dtype=torch.bfloat16, device="cpu"):
    if w.paged:
        return make_paged(w.seqlens_q, w.seqlens_k, w.page_size, w.Hq, w.Hkv, w.d, w.seed, dtype, device=device)
    return make_varlen(w.seqlens_q, w.seqlens_k, w.Hq, w.Hkv, w.d, w.seed, dtype, device=device)


def _lengths_to_total(total, lo, hi, seed):
    """Log-uniform lengths in [lo, hi] (seeded) until they sum to at least `total`; the last
    one is cut so that the sum is exactly `total`."""
    out, s, k = [], 0, 0
    while s < total:
        n = _lengths(1, lo, hi, seed * 1000 + k)[0]
        n = min(n, total - s)
        out.append(n)
        s += n
        k += 1
    return tuple(out)


def bench_var_workloads():
    """Throughput-size serving batches (about 32k query tokens for prefill)."""
    L1 = _lengths_to_total(32768, 256, 8192, 61)
    L2 = _lengths_to_total(32768, 256, 8192, 62)
    Lk = _lengths(128, 1024, 32768, 63)
    g = torch.Generator(device="cpu")
    g.manual_seed(64)
    Lq = tuple(int(x) for x in torch.randint(1, 17, (128,), generator=g))
    return [VarWorkload("varlen_prefill_32k_hd128", L1, L1, 16, 4, 128, 61),
            VarWorkload("paged_prefill_32k_hd256", L2, L2, 8, 8, 256, 62, paged=True, page_size=128),
            VarWorkload("paged_decode_128seq_hd256", Lq, Lk, 8, 8, 256, 63, paged=True, page_size=128,
                        causal_modes=(True,))]
