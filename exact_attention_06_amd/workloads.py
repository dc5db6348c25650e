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
    8 query heads, batch sized to about 32k tokens, sequence lengths 1k..128k.
The head_dim=128 sweep (16 query heads, MHA and 4:1 GQA) and the spiked-key video
shape (every 16th key scaled by 4, to make peaked softmax rows) are synthetic
stand-ins with the same structure; there is no dataset behind any of them.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import torch

__all__ = ["Workload", "make_qkv", "sample_rows", "tiny", "ragged", "hd128_sweep",
           "hd256_sweep", "video", "all_workloads", "by_name"]

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


def video():
    return Workload("video", B=1, N=20480, Hq=56, Hkv=56, d=128, seed=5, causal_modes=(False,),
                    k_spike=True, full_oracle=False)


def all_workloads():
    return [tiny(), ragged()] + hd128_sweep() + hd256_sweep() + [video()]


def by_name(name):
    for w in all_workloads():
        if w.name == name:
            return w
    raise KeyError(name)


def inputs_for(w: Workload, dtype=torch.bfloat16):
    return make_qkv(w.B, w.N, w.N, w.Hq, w.Hkv, w.d, w.seed, dtype=dtype, k_spike=w.k_spike)
