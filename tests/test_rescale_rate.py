"""How often the lazy rescale fires (CPU emulation of the per-wave rule, test infrastructure only).

The pages report that rescaling only when the row maximum grows "significantly" cuts rescale
work about tenfold (Dutch page, section "Slimmere Online Softmax-herwaardering"). The kernels
decide per wave of 32 query rows and per key tile: they rescale when some row's tile maximum
(log2 units, c = scale * log2 e) exceeds its running maximum by more than TAU = 8. This module
replays that rule on fp32 scores of seeded workloads (the first tile of a wave always sets the
maximum and is not counted) and checks that TAU = 8 rescales far less often than TAU = 0.
`python tests/test_rescale_rate.py` prints the rates for the video shape and hd256 at N = 8192.
"""

import math

import numpy as np
import torch

from exact_attention_06_amd import workloads as W


def wave_rescale_fraction(q, k, scale, bc, tau, causal=False, waves=None, seed=0):
    """Fraction of (wave, key tile) steps after the first tile that rescale.

    q: [N, d] and k: [N, d] fp32 for one (batch, head); waves of 32 rows; key tiles of bc keys.
    """
    n = q.shape[0]
    c = scale * math.log2(math.e)
    nw = (n + 31) // 32
    g = np.random.default_rng(seed)
    pick = range(nw) if waves is None else g.choice(nw, size=min(waves, nw), replace=False)
    steps = fired = 0
    for w in pick:
        r0, r1 = 32 * w, min(n, 32 * w + 32)
        s = (q[r0:r1] @ k.T).numpy().astype(np.float32) * np.float32(c)     # [rows, N] log2 units
        if causal:
            j = np.arange(n)[None, :]
            s = np.where(j <= np.arange(r0, r1)[:, None], s, -np.inf)
        last = r1 if causal else n
        m = None
        for t0 in range(0, last, bc):
            mt = s[:, t0:t0 + bc].max(axis=1)
            if m is None:
                m = mt
                continue
            steps += 1
            if np.any(mt > m + tau):
                fired += 1
                m = np.maximum(m, mt)
    return fired / max(steps, 1)


def _one_head(w, b=0, h=0):
    q, k, _ = W.make_qkv(1, w.N, w.N, w.Hq, w.Hkv, w.d, w.seed + b, dtype=torch.float32, k_spike=w.k_spike)
    return q[0, :, h], k[0, :, h // (w.Hq // w.Hkv)]


def test_threshold_cuts_rescales():
    w = W.Workload("spiked", B=1, N=2048, Hq=1, Hkv=1, d=128, seed=9, k_spike=True)
    q, k = _one_head(w)
    f0 = wave_rescale_fraction(q, k, w.scale, 64, 0.0)
    f8 = wave_rescale_fraction(q, k, w.scale, 64, 8.0)
    assert f8 <= f0 / 4, (f0, f8)
    assert 0.0 <= f8 <= 1.0


def test_no_rescale_without_growth():
    # identical keys: every tile has the same maximum, so after the first tile nothing fires
    q = torch.randn(64, 16, generator=torch.Generator().manual_seed(1))
    k = torch.randn(1, 16, generator=torch.Generator().manual_seed(2)).repeat(512, 1)
    assert wave_rescale_fraction(q, k, 0.25, 32, 0.0) == 0.0


if __name__ == "__main__":
    for w, bc in ((W.video(), 64), (W.by_name("hd256_N8192"), 32), (W.by_name("hd128_N8192_mha"), 64)):
        q, k = _one_head(w)
        for tau in (0.0, 8.0):
            f = wave_rescale_fraction(q, k, w.scale, bc, tau, waves=64)
            print(f"{w.name:18s} key tile {bc:3d}  tau={tau:3.0f}: {100 * f:5.1f}% of (wave, tile) steps rescale")
