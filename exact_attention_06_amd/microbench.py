"""Measurement tools behind the performance analysis (not part of the library's path).

* MFMA issue rate with LDS fragment reads: csrc/ubench_mfma_lds.hip interleaves
  v_mfma_f32_32x32x16_bf16 with the hd256 forward kernel's own K (ds_read_b128) and V^T
  (ds_read_b64_tr_b16) fragment reads at 1 KB and 0.5 KB per MFMA, eight waves per CU on every
  CU, and reports each mix's MFMA rate against MFMA issue alone.
* Shader clock under load: runs a workload back to back for a few seconds (that MFMA loop,
  the platform bf16 GEMM, or the forward pass on a benchmark workload) and samples the clock
  with rocm-smi in a child process.

    python -m exact_attention_06_amd.microbench --build          # compile (no GPU needed)
    python -m exact_attention_06_amd.microbench [--clock-seconds 6] [--out FILE]
"""

from __future__ import annotations

import argparse
import ctypes
import os
import re
import subprocess
import sys
import threading
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "ubench_mfma_lds.hip")
LIB = os.path.join(PKG, "libubench_mfma_lds.so")

MODES = {
    0: "MFMA only",
    1: "MFMA + K fragments (ds_read_b128), 1 KB per MFMA",
    2: "MFMA + V^T fragments (ds_read_b64_tr_b16), 1 KB per MFMA",
    3: "MFMA + K fragments, 0.5 KB per MFMA",
    4: "MFMA + V^T fragments, 0.5 KB per MFMA",
}


def build() -> str:
    from .build import HIPCC_FLAGS, hipcc

    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    flags = [f for f in HIPCC_FLAGS if not f.startswith("-I") and not f.startswith(os.sep)]
    cmd = [hipcc()] + flags + [SRC, "-o", LIB]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{res.stderr[-2000:]}")
    return LIB


def _cus() -> int:
    import torch

    return torch.cuda.get_device_properties(0).multi_processor_count


def mfma_lds_table(iters: int = 20000):
    import torch

    lib = ctypes.CDLL(LIB)
    blocks = _cus()
    out = torch.zeros(blocks * 512, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    rows = []
    for mode in MODES:
        run = lambda: lib.ub_run(mode, ctypes.c_void_p(out.data_ptr()), iters, blocks, ctypes.c_void_p(st))
        assert run() == 0
        torch.cuda.synchronize()
        best = 1e9
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            assert run() == 0
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1))
        flops = blocks * 8 * lib.ub_mfmas_per_iter(mode) * iters * 32768.0
        rows.append((mode, flops / (best * 1e-3) / 1e12))
    base = rows[0][1]
    return [(MODES[m], tf, tf / base) for m, tf in rows]


def _sample_clock(stop, samples):
    while not stop.is_set():
        try:
            res = subprocess.run(["rocm-smi", "-g"], capture_output=True, text=True, timeout=10)
            samples += [int(x) for x in re.findall(r"\((\d+)Mhz\)", res.stdout)]
        except (OSError, subprocess.TimeoutExpired):
            return
        time.sleep(0.5)


def clock_under_load(seconds: float):
    import torch

    from . import forward
    from . import workloads as W

    lib = ctypes.CDLL(LIB)
    blocks = _cus()
    out = torch.zeros(blocks * 512, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    loads = []
    iters = 100000
    loads.append(("MFMA only (the loop above, mode 0)",
                  lambda: lib.ub_run(0, ctypes.c_void_p(out.data_ptr()), iters, blocks, ctypes.c_void_p(st)),
                  blocks * 8 * 2 * iters * 32768.0))
    a = torch.randn((8192, 8192), device="cuda", dtype=torch.bfloat16)
    b = torch.randn((8192, 8192), device="cuda", dtype=torch.bfloat16)
    loads.append(("torch.mm bf16 8192 x 8192 x 8192 (platform GEMM)", lambda: torch.mm(a, b), 2.0 * 8192 ** 3))
    for name in ("hd256_N8192", "hd128_N8192_mha"):
        w = W.by_name(name)
        q, k, v = (x.cuda() for x in W.make_qkv(w.B, w.N, w.N, w.Hq, w.Hkv, w.d, w.seed))
        loads.append((f"fa.forward {name} non-causal", lambda q=q, k=k, v=v: forward(q, k, v), w.flops(False)))
    rows = []
    for name, run, flops in loads:
        run()
        torch.cuda.synchronize()
        stop, samples = threading.Event(), []
        t0 = time.time()
        n, best = 0, 1e9
        sampler = None
        while time.time() - t0 < seconds:
            if sampler is None and time.time() - t0 > seconds / 3:
                sampler = threading.Thread(target=_sample_clock, args=(stop, samples))
                sampler.start()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(10):
                run()
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) / 10)
            n += 10
        stop.set()
        if sampler is not None:
            sampler.join()
        mhz = sorted(samples)[len(samples) // 2] if samples else None
        rows.append((name, flops / (best * 1e-3) / 1e12, mhz))
        print(f"[clock] {name}: {rows[-1][1]:.1f} TFLOP/s, sclk {mhz} MHz", flush=True)
    return rows


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--clock-seconds", type=float, default=6.0, help="0: skip the clock measurement")
    ap.add_argument("--out", default="")
    ap.add_argument("--build", action="store_true", help="compile the microbenchmark and exit")
    a = ap.parse_args(argv)
    if a.build:
        print(build())
        return
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is not built: python -m exact_attention_06_amd.microbench --build")
    lines = ["| mix (8 waves per CU, every CU) | TFLOP/s | MFMA rate vs MFMA only |", "|---|---|---|"]
    for name, tf, rel in mfma_lds_table():
        lines.append(f"| {name} | {tf:.0f} | {rel:.2f} |")
        print(f"[ubench] {name}: {tf:.0f} TFLOP/s ({rel:.2f})", flush=True)
    if a.clock_seconds > 0:
        lines += ["", "| workload | TFLOP/s | median sclk (MHz) |", "|---|---|---|"]
        for name, tf, mhz in clock_under_load(a.clock_seconds):
            lines.append(f"| {name} | {tf:.0f} | {mhz if mhz else 'n/a'} |")
    text = "\n".join(lines) + "\n"
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    print(text)


if __name__ == "__main__":
    sys.exit(main())
