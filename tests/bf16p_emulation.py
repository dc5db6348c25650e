"""CPU model of the forward kernel's rounding, for the error-tail analysis of peaked rows.

Not the oracle (that is the fp64 definition in oracle/): this script replays, in numpy, the
arithmetic the hd128 kernel performs for one head, wave by wave, to show where its O error
comes from. Per 32-row wave and 64-key tile it takes fp32 scores, the causal mask, the row max
in log2 units, the per-wave lazy rescale (every row of the wave is rescaled when one row's tile
max exceeds its running max by more than tau), p = exp2(c s - m) in fp32, P rounded to bf16
(RNE), the fp32 row sums (of p for the LSE, of the rounded P for O), P.V with fp32
accumulation, the hi + lo split of the first tile of a block whose rows see fewer than 512
keys, and O = acc / sum rounded to bf16. Blocks are 256 query rows (the 8-wave form).

    python tests/bf16p_emulation.py            # the table behind the peaked-row reading

prints, for the spiked-key stress shapes, how many elements with |O_ref| < 4 land above 1e-2
for tau = 8, 4, 2 and 0 (0: the running max always exact).
"""

import os
import sys

import numpy as np
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

from exact_attention_06_amd import workloads as W  # noqa: E402
from oracle import attention_ref  # noqa: E402

F32 = np.float32
LOG2E = F32(1.4426950408889634)


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


def emulate_head(Q, K, V, scale, causal, tau, BR=256, BC=64, split_keys=512):
    """Q [N, d], K/V [Nk, d] (fp32 copies of bf16 values) -> bf16-rounded O [N, d] as fp32."""
    N, d = Q.shape
    Nk = K.shape[0]
    c = F32(scale) * LOG2E
    out = np.zeros((N, d), F32)
    for r0 in range(0, N, 32):
        blk0 = (r0 // BR) * BR
        nw = min(32, N - r0)
        rows = r0 + np.arange(32)
        Qw = np.zeros((32, d), F32)
        Qw[:nw] = Q[r0:r0 + nw]
        last_key = min(Nk, blk0 + BR) if causal else Nk
        split_first = (min(Nk, blk0 + 1) if causal else Nk) < split_keys
        m = np.full(32, -np.inf, F32)
        lO = np.zeros(32, F32)
        acc = np.zeros((32, d), F32)
        for t in range((last_key + BC - 1) // BC):
            ks = np.arange(t * BC, (t + 1) * BC)
            if causal and rows[-1] < ks[0]:
                continue  # every row of the wave precedes the tile
            valid = ks < Nk
            Kt = np.zeros((BC, d), F32)
            Vt = np.zeros((BC, d), F32)
            Kt[valid] = K[ks[valid]]
            Vt[valid] = V[ks[valid]]
            S = (Qw.astype(np.float64) @ Kt.T.astype(np.float64)).astype(F32)
            mask = ~valid[None, :]
            if causal:
                mask = mask | (ks[None, :] > rows[:, None])
            S = np.where(mask, -np.inf, S).astype(F32)
            mt = (S.max(axis=1) * c).astype(F32)
            if (mt > m + F32(tau)).any():
                mnew = np.maximum(m, mt)
                with np.errstate(invalid="ignore"):
                    alpha = np.exp2((m - mnew).astype(F32)).astype(F32)
                alpha = np.where(np.isneginf(m), F32(0), alpha)
                acc = (acc * alpha[:, None]).astype(F32)
                lO = (lO * alpha).astype(F32)
                m = mnew
            negm = np.where(np.isneginf(m), F32(0), -m).astype(F32)
            p = np.exp2((S * c + negm[:, None]).astype(F32)).astype(F32)
            pb = _bf16(p)
            parts = [pb, _bf16(p - pb)] if (t == 0 and split_first) else [pb]
            for pp in parts:
                lO = (lO + pp.sum(axis=1, dtype=F32)).astype(F32)
                acc = (acc + (pp.astype(np.float64) @ Vt.astype(np.float64)).astype(F32)).astype(F32)
        out[r0:r0 + nw] = _bf16(acc / lO[:, None])[:nw]
    return out


def tail(B, N, H, d, seed, causal, tau, spike=True):
    """(elements with |O_ref| < 4 above 1e-2, their largest error, elements compared)."""
    q, k, v = W.make_qkv(B, N, N, H, H, d, seed, k_spike=spike)
    scale = float(torch.tensor(d ** -0.5, dtype=torch.float32))
    O_ref, _ = attention_ref(q, k, v, causal, scale)
    over, worst = 0, 0.0
    for b in range(B):
        for h in range(H):
            o = emulate_head(q[b, :, h].float().numpy(), k[b, :, h].float().numpy(), v[b, :, h].float().numpy(),
                             scale, causal, tau)
            ref = O_ref[b, :, h]
            err = np.abs(o - ref)[np.abs(ref) < 4]
            over += int((err > 1e-2).sum())
            worst = max(worst, float(err.max()))
    return over, worst, O_ref.size


def main():
    shapes = [("causal, 96 heads x 768 rows", 1, 768, 96, True, (50, 51, 52, 53)),
              ("non-causal, 48 heads x 1536 rows", 1, 1536, 48, False, (60, 61))]
    print("| shape (hd128, every 16th key x4) | seed | tau = 8 | tau = 4 | tau = 2 | tau = 0 |")
    print("|---|---|---|---|---|---|")
    for name, B, N, H, causal, seeds in shapes:
        for seed in seeds:
            cells = []
            for tau in (8.0, 4.0, 2.0, 0.0):
                over, worst, _ = tail(B, N, H, 128, seed, causal, tau)
                cells.append(f"{over} (max {worst:.3e})")
            print(f"| {name} | {seed} | " + " | ".join(cells) + " |", flush=True)


if __name__ == "__main__":
    main()
