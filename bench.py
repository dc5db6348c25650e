#!/usr/bin/env python3
"""Forward-attention throughput on one MI355X: TFLOPS and fraction of the dense bf16 MFMA peak.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--causal] [--no-sweep]

A step is one forward pass (one fa_fwd launch) over the named workload, inputs already
resident in HBM. FLOPs = 4*B*Hq*Nq*Nk*d, halved for causal. Prints ONE JSON line on stdout;
a table of the head_dim 128/256 sweep goes to stderr (and into the JSON as "sweep").

The CPU baseline is the fp64 oracle timed on this host's cores over a bounded sample of
query rows of the same workload (a reported baseline, not the target).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0  # MI355X dense fp8 MFMA
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16/fp16 MFMA peak (published)
PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E (published)
DEFAULT_WORKLOAD = "hd256_N8192"
PAGES_B200 = {  # pages' own forward TFLOPS for the hd256 snapshot workloads (B200, context only)
    ("hd256_N1024", False): 950, ("hd256_N2048", False): 1280, ("hd256_N4096", False): 1477,
    ("hd256_N8192", False): 1594, ("hd256_N16384", False): 1663, ("hd256_N32768", False): 1709,
    ("hd256_N65536", False): 1562, ("hd256_N131072", False): 1481,
    ("hd256_N1024", True): 584, ("hd256_N2048", True): 897, ("hd256_N4096", True): 1191,
    ("hd256_N8192", True): 1385, ("hd256_N16384", True): 1505, ("hd256_N32768", True): 1589,
    ("hd256_N65536", True): 1594, ("hd256_N131072", True): 1457,
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


from exact_attention_06_amd.profile_summary import kernel_source_hash  # noqa: E402


def gpu_inputs(w, torch):
    """Seeded N(0,1) draws made on the GPU (same recipe as the CPU generator: fp32 normal,
    rounded to bf16, optional x4 on every 16th key); used for timing only."""
    g = torch.Generator(device="cuda")
    g.manual_seed(w.seed)
    dev = "cuda"
    q = torch.randn((w.B, w.N, w.Hq, w.d), generator=g, device=dev).to(torch.bfloat16)
    k = torch.randn((w.B, w.N, w.Hkv, w.d), generator=g, device=dev).to(torch.bfloat16)
    v = torch.randn((w.B, w.N, w.Hkv, w.d), generator=g, device=dev).to(torch.bfloat16)
    if w.k_spike:
        k[:, 0::16] *= 4
    return q, k, v


def time_forward(fa, torch, q, k, v, causal, scale, steps, warmup):
    """Returns (ms_per_step, per-launch ms list) with HIP events on the launch stream."""
    out = torch.empty_like(q)
    lse = torch.empty((q.shape[0], q.shape[2], q.shape[1]), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fa.forward(q, k, v, causal=causal, scale=scale, out=out, lse=lse)
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record(stream)
    for i in range(steps):
        fa.forward(q, k, v, causal=causal, scale=scale, out=out, lse=lse)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    total = evs[0].elapsed_time(evs[-1])
    return total / steps, per


def cpu_baseline(w, causal, budget_s=12.0):
    """Time the fp64 oracle on a bounded sample of query rows of workload w.

    Rows are taken in chunks of 256 seeded random query rows per (batch, head), walking over
    the heads of each batch in turn (and over them again with fresh rows) until about
    `budget_s` seconds of CPU work have been done; FLOPs are counted as 4*d per visible key
    per row.
    """
    import numpy as np
    import torch

    from exact_attention_06_amd import workloads as W
    from oracle import attention_ref

    # the host cores this process may run on; the BLAS pool behind numpy is set to that many
    # threads for the timed oracle calls
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limiter = threadpool_limits(limits=cores, user_api="blas")
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
                           or [cores])
    except Exception:  # pragma: no cover
        limiter, blas_threads = None, cores
    R = 256
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed + 200)
    dt = 0.0  # seconds spent inside the oracle (input generation is not timed)
    done_rows = 0
    flops = 0.0
    heads = 0
    inputs = {}
    while dt <= budget_s:
        for b in range(w.B):
            if b not in inputs:
                inputs = {b: W.make_qkv(1, w.N, w.N, w.Hq, w.Hkv, w.d, w.seed + b, k_spike=w.k_spike)}
            q, k, v = inputs[b]
            for h in range(w.Hq):
                kvh = h // (w.Hq // w.Hkv)
                rows = torch.randint(0, w.N, (1, 1, R), generator=g).numpy()
                t0 = time.perf_counter()
                attention_ref(q[:, :, h:h + 1], k[:, :, kvh:kvh + 1], v[:, :, kvh:kvh + 1], causal, w.scale,
                              rows=rows)
                dt += time.perf_counter() - t0
                done_rows += R
                heads += 1
                vis = (rows[0, 0] + 1) if causal else np.full(R, w.N)
                flops += float(np.sum(4.0 * vis * w.d))
                if dt > budget_s:
                    break
            if dt > budget_s:
                break
    if limiter is not None:
        limiter.restore_original_limits()
    return {"value": flops / dt / 1e12, "unit": "TFLOPS", "cores": int(cores), "blas_threads": int(blas_threads),
            "kind": "oracle",
            "sample": f"{done_rows} random query rows ({R} per (batch, head), {heads} (batch, head) visits) of {w.name} "
                      f"{'causal' if causal else 'non-causal'} with all {w.N} keys, fp64 numpy oracle; "
                      f"{dt:.1f} s of CPU work; FLOPs 4*d per visible key per row"}


def load_profile(kernel_name):
    """The committed rocprofv3 record of this kernel (profiles/traffic.json), or None when the
    kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    e = rec.get(kernel_name)
    if not e or e.get("source_hash") != kernel_source_hash():
        return None
    return e


def load_traffic(kernel_name):
    e = load_profile(kernel_name)
    return None if e is None else e.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--causal", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--sweep-steps", type=int, default=6)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--only-fp8", action="store_true",
                    help="besides the headline workload, run only the fp8 section; used to profile it")
    ap.add_argument("--only-variants", action="store_true",
                    help="besides the headline workload, run only the serving variants (packed and "
                         "paged prefill, paged decode); used to profile them")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (HBM counter calibration)")
    ap.add_argument("--gemm-n", type=int, default=0,
                    help="only time torch.matmul on two n x n bf16 matrices (the platform GEMM's "
                         "MFMA throughput on this board, for context)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU mode "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_attention_06_amd as fa
    from exact_attention_06_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)

    if args.copy_mib:
        # A plain copy of known size: HBM counters read over it calibrate FETCH_SIZE/WRITE_SIZE.
        n = args.copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_mib": args.copy_mib, "bytes_read": n, "bytes_written": n,
                          "launches": max(1, args.steps)}), flush=True)
        return

    if args.gemm_n:
        # The platform's own dense bf16 GEMM (hipBLASLt behind torch.matmul) under the same
        # board power limit: a practical ceiling for MFMA-bound kernels, reported beside the
        # published peak.
        n = args.gemm_n
        g = torch.Generator(device="cuda")
        g.manual_seed(0)
        a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
        b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
        for _ in range(max(1, args.warmup)):
            c = a @ b
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        reps = max(1, args.steps)
        e0.record()
        for _ in range(reps):
            c = a @ b
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        tf = 2 * n ** 3 / (ms * 1e-3) / 1e12
        print(json.dumps({"gemm_n": n, "dtype": "bf16", "ms": round(ms, 4), "tflops": round(tf, 1),
                          "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4), "launches": reps}), flush=True)
        del c
        return

    w = W.by_name(args.workload)
    causal = bool(args.causal)
    q, k, v = gpu_inputs(w, torch)
    torch.cuda.synchronize()
    ms, per = time_forward(fa, torch, q, k, v, causal, w.scale, args.steps, args.warmup)
    flops = w.flops(causal)
    tflops = flops / (ms * 1e-3) / 1e12
    avg_launch_ms = sum(per) / len(per)
    median_launch_ms = sorted(per)[len(per) // 2]
    achieved = flops / (avg_launch_ms * 1e-3) / 1e12
    del q, k, v
    torch.cuda.empty_cache()
    log(f"[bench] {w.name} causal={causal}: {ms:.3f} ms/step, {tflops:.1f} TFLOPS "
        f"({100 * tflops / PEAK_BF16_TFLOPS:.1f}% of {PEAK_BF16_TFLOPS:.0f})")

    rest = not args.no_sweep and not args.only_variants and not args.only_fp8  # sweep, short, fp8
    sweep = []
    if rest:
        pts = [x for x in W.hd128_sweep() + W.hd256_sweep() + [W.video()] + W.hd512_sweep()]
        for x in pts:
            qx, kx, vx = gpu_inputs(x, torch)
            for c in x.causal_modes:
                m, _ = time_forward(fa, torch, qx, kx, vx, c, x.scale, args.sweep_steps, 2)
                t = x.flops(c) / (m * 1e-3) / 1e12
                ent = {"workload": x.name, "causal": c, "B": x.B, "N": x.N, "Hq": x.Hq, "Hkv": x.Hkv,
                       "d": x.d, "ms": round(m, 4), "tflops": round(t, 1),
                       "frac_peak": round(t / PEAK_BF16_TFLOPS, 4)}
                b200 = PAGES_B200.get((x.name, c))
                if b200:
                    ent["pages_b200_tflops"] = b200
                sweep.append(ent)
                log(f"[sweep] {x.name:20s} {'causal' if c else 'noncausal':9s} {m:8.3f} ms "
                    f"{t:7.1f} TFLOPS {100 * t / PEAK_BF16_TFLOPS:5.1f}%")
            del qx, kx, vx
            torch.cuda.empty_cache()

    # backward pass (gradients of sum(O * dO)); FLOPs counted as 2.5x the forward's
    # (five N x N x d products), the usual convention
    backward = []
    if not args.no_backward and not args.only_variants and not args.only_fp8:
        for name in ("hd128_N8192_mha", "hd256_N8192"):
            x = W.by_name(name)
            qx, kx, vx = gpu_inputs(x, torch)
            g = torch.Generator(device="cuda")
            g.manual_seed(x.seed + 7)
            dox = torch.randn(qx.shape, generator=g, device="cuda").to(torch.bfloat16)
            for c in (False, True):
                o, lse = fa.forward(qx, kx, vx, causal=c, scale=x.scale)
                for _ in range(2):
                    fa.backward(qx, kx, vx, o, lse, dox, causal=c, scale=x.scale)
                torch.cuda.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                n = max(1, args.sweep_steps)
                e0.record()
                for _ in range(n):
                    fa.backward(qx, kx, vx, o, lse, dox, causal=c, scale=x.scale)
                e1.record()
                torch.cuda.synchronize()
                m = e0.elapsed_time(e1) / n
                t = 2.5 * x.flops(c) / (m * 1e-3) / 1e12
                backward.append({"workload": x.name, "causal": c, "ms": round(m, 4), "tflops": round(t, 1),
                                 "frac_peak": round(t / PEAK_BF16_TFLOPS, 4)})
                log(f"[bwd] {x.name:20s} {'causal' if c else 'noncausal':9s} {m:8.3f} ms {t:7.1f} TFLOPS")
            del qx, kx, vx, dox, o, lse
            torch.cuda.empty_cache()

    # short sequences, few heads: the plain grid vs split-KV (the library's split count)
    short = []
    if rest:
        for (B_, N_, H_, d_) in ((1, 1024, 8, 256), (2, 1024, 8, 256), (1, 2048, 8, 256), (1, 1024, 16, 128)):
            g = torch.Generator(device="cuda")
            g.manual_seed(71)
            qx = torch.randn((B_, N_, H_, d_), generator=g, device="cuda").to(torch.bfloat16)
            kx = torch.randn((B_, N_, H_, d_), generator=g, device="cuda").to(torch.bfloat16)
            vx = torch.randn((B_, N_, H_, d_), generator=g, device="cuda").to(torch.bfloat16)
            for c in (False, True):
                fl = 4.0 * B_ * H_ * N_ * N_ * d_ / (2 if c else 1)
                ns = fa.num_splits(B_, N_, N_, H_, d_, c)
                res = {}
                modes = [("plain", lambda: fa.forward(qx, kx, vx, causal=c))]
                if ns > 1:  # with one split the library's choice is the plain grid
                    modes.append(("splitkv", lambda: fa.forward_splitkv(qx, kx, vx, causal=c, num_splits=ns)))
                for mode, fn in modes:
                    for _ in range(3):
                        fn()
                    torch.cuda.synchronize()
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    n = 50  # launches of tens of microseconds
                    e0.record()
                    for _ in range(n):
                        fn()
                    e1.record()
                    torch.cuda.synchronize()
                    res[mode] = e0.elapsed_time(e1) / n
                res.setdefault("splitkv", res["plain"])
                ent = {"B": B_, "N": N_, "Hq": H_, "d": d_, "causal": c, "splits": ns,
                       "library_choice": "plain grid" if ns == 1 else f"split-KV x{ns}",
                       "plain_ms": round(res["plain"], 4), "splitkv_ms": round(res["splitkv"], 4),
                       "plain_tflops": round(fl / (res["plain"] * 1e-3) / 1e12, 1),
                       "splitkv_tflops": round(fl / (res["splitkv"] * 1e-3) / 1e12, 1)}
                short.append(ent)
                log(f"[short] B={B_} N={N_} Hq={H_} d={d_} {'causal' if c else 'noncausal':9s} plain "
                    f"{ent['plain_tflops']:7.1f} TFLOPS, library choice ({ent['library_choice']}) "
                    f"{ent['splitkv_tflops']:7.1f} TFLOPS")

    # fp8 (e4m3) inputs, one dequantisation factor per tensor, bf16 output; priced against the
    # fp8 MFMA peak
    fp8 = []
    if rest or args.only_fp8:
        for name in ("hd128_N8192_mha", "hd256_N8192"):
            x = W.by_name(name)
            qx, kx, vx = gpu_inputs(x, torch)
            sc = [float(t.abs().max()) / 224.0 for t in (qx, kx, vx)]
            q8, k8, v8 = ((t.float() / s_).to(torch.float8_e4m3fn) for t, s_ in zip((qx, kx, vx), sc))
            del qx, kx, vx
            for c in (False, True):
                call = lambda: fa.forward_fp8(q8, k8, v8, sc[0], sc[1], sc[2], causal=c, scale=x.scale)
                # this section follows the short split-KV launches, during which the shader clock
                # drops: 10 warm-up launches, then the mean of 3 repeats of the timed launches
                for _ in range(10):
                    call()
                torch.cuda.synchronize()
                n = max(1, args.sweep_steps)
                reps = []
                for _ in range(3):
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record()
                    for _ in range(n):
                        call()
                    e1.record()
                    torch.cuda.synchronize()
                    reps.append(e0.elapsed_time(e1) / n)
                m = sum(reps) / len(reps)
                t = x.flops(c) / (m * 1e-3) / 1e12
                fp8.append({"workload": x.name, "causal": c, "ms": round(m, 4), "tflops": round(t, 1),
                            "frac_fp8_peak": round(t / PEAK_FP8_TFLOPS, 4)})
                log(f"[fp8] {x.name:20s} {'causal' if c else 'noncausal':9s} {m:8.3f} ms {t:7.1f} TFLOPS "
                    f"{100 * t / PEAK_FP8_TFLOPS:5.1f}% of {PEAK_FP8_TFLOPS:.0f}")
            del q8, k8, v8
            torch.cuda.empty_cache()

    # serving variants: packed variable-length prefill, paged prefill, paged decode; each without
    # splits and, where the library picks a split count for its shape, split over the keys too
    variants = []
    if (not args.no_sweep or args.only_variants) and not args.only_fp8:
        for x in W.bench_var_workloads():
            mq = max(x.seqlens_q)
            if x.paged:
                qx, kc, vc, cu, used, bt = (t.cuda() for t in W.var_inputs(x, device="cuda"))
                bound = bt.shape[1] * kc.shape[1]
                call = lambda c, ns: fa.forward_paged(qx, kc, vc, cu, used, bt, mq, causal=c, scale=x.scale,
                                                      num_splits=ns)
            else:
                qx, kx, vx, cu, cuk = (t.cuda() for t in W.var_inputs(x, device="cuda"))
                bound = kx.shape[0]
                call = lambda c, ns: fa.forward_varlen(qx, kx, vx, cu, cuk, mq, causal=c, scale=x.scale,
                                                       num_splits=ns)
            ns_lib = fa.var_num_splits(x.B, mq, bound, x.Hq, x.d)
            for c in x.causal_modes:
                for ns in [0] + ([ns_lib] if ns_lib else []):
                    for _ in range(2):
                        call(c, ns)
                    torch.cuda.synchronize()
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    n = max(1, args.sweep_steps)
                    e0.record()
                    for _ in range(n):
                        call(c, ns)
                    e1.record()
                    torch.cuda.synchronize()
                    m = e0.elapsed_time(e1) / n
                    t = x.flops(c) / (m * 1e-3) / 1e12
                    kv_bytes = 2 * 2 * x.Hkv * x.d * sum(x.seqlens_k)  # K and V rows used, bf16
                    ent = {"workload": x.name, "causal": c, "B": x.B, "total_q": sum(x.seqlens_q),
                           "total_k": sum(x.seqlens_k), "Hq": x.Hq, "Hkv": x.Hkv, "d": x.d, "paged": x.paged,
                           "num_splits": ns, "ms": round(m, 4), "tflops": round(t, 1),
                           "kv_gbps": round(kv_bytes / (m * 1e-3) / 1e9, 1),
                           "kv_frac_hbm_peak": round(kv_bytes / (m * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}
                    variants.append(ent)
                    log(f"[var] {x.name:26s} {'causal' if c else 'noncausal':9s} splits {ns:2d} {m:8.3f} ms "
                        f"{t:7.1f} TFLOPS K/V {ent['kv_gbps']:7.1f} GB/s")
            torch.cuda.empty_cache()

    cpu = None if args.no_cpu_baseline else cpu_baseline(w, causal)
    if cpu:
        log(f"[cpu] oracle {cpu['value'] * 1e3:.2f} GFLOP/s on {cpu['cores']} cores, {cpu['blas_threads']} BLAS "
            f"threads ({cpu['sample']})")

    kname = f"fwd_kernel<{w.d},{'causal' if causal else 'noncausal'},bf16>"
    # counter figures from the same committed profile as `traffic` (null when stale): the shader
    # clock the kernel ran at and its MFMA/VALU busy fractions
    prof = load_profile(kname)
    counters = None if prof is None or "sclk_ghz" not in prof else {
        "sclk_ghz": prof["sclk_ghz"], "mfma_busy": prof["mfma_busy"], "valu_busy": prof["valu_busy"],
        "source": "profiles/traffic.json (rocprofv3 SQ counters)"}
    b200 = PAGES_B200.get((w.name, causal))
    rec = {
        "metric": "fwd attention TFLOPS + % of MI355X bf16 MFMA peak, hd128/hd256 at N=1k-128k",
        "value": round(tflops, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(tflops / b200, 4) if b200 else None,
        "dtype": "bf16",
        "data": "synthetic: seeded i.i.d. N(0,1) fp32 draws rounded to bf16",
        "config": {"workload": w.name, "B": w.B, "Nq": w.N, "Nk": w.N, "Hq": w.Hq, "Hkv": w.Hkv,
                   "d": w.d, "causal": causal, "scale": w.scale, "tokens": w.B * w.N,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": load_traffic(kname), "kernel": kname,
                     "counters": counters,
                     "avg_launch_ms": round(avg_launch_ms, 4),
                     "median_launch_ms": round(median_launch_ms, 4),
                     "flops_per_launch": flops},
        "cpu_baseline": cpu,
        "sweep": sweep,
        "backward": backward,
        "variants": variants,
        "short_splitkv": short,
        "fp8": fp8,
        "kernel_source_hash": kernel_source_hash(),
    }
    if b200:
        rec["vs_baseline_note"] = (f"ratio to the pages' B200 figure for this workload ({b200} TFLOPS, "
                                   "another machine: context, not the target)")
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
