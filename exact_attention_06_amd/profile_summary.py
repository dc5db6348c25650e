"""Summaries of rocprofv3 runs of the forward kernel, for profiles/ and bench.py.

    python -m exact_attention_06_amd.profile_summary --name 'fwd_kernel<256,noncausal,bf16>' \
        --kernel-regex 'fwd_kernel<256, false, fa::Bf16, 0' --workload hd256_N8192 --skip 5 \
        --trace DIR --pmc DIR [--pmc DIR ...] --cmd '...' [--cmd '...'] \
        --out profiles/NAME.md --traffic-json profiles/traffic.json

Each DIR is the output directory of one rocprofv3 run (`--output-format csv`) of the same
command: `--kernel-trace --stats` for --trace, one `--pmc` counter set for each --pmc. Only the
dispatches of the named kernel count, in launch order, and the first --skip of them (the
command's warm-up launches) are dropped, so the averages cover the timed launches only.

HBM traffic = FETCH_SIZE x fetch factor + WRITE_SIZE x write factor (KiB -> bytes), with the
factors that the same counters give for a plain device copy of known size (1 GiB:
FETCH_SIZE reads 0.5 KiB per KiB read, WRITE_SIZE 1.0).
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBPS = 8000.0
FETCH_FACTOR = 2.0  # bytes read per FETCH_SIZE byte (1 GiB copy calibration)
WRITE_FACTOR = 1.0
NUM_XCD, NUM_CU, NUM_SIMD = 8, 256, 1024


def kernel_source_hash() -> str:
    """Hash of the HIP sources (csrc/): a profile is current only for the sources it was
    taken on."""
    h = hashlib.sha256()
    cdir = os.path.join(PKG, "csrc")
    for n in sorted(os.listdir(cdir)):
        with open(os.path.join(cdir, n), "rb") as f:
            h.update(n.encode() + f.read())
    return h.hexdigest()[:16]


def _norm(k: str) -> str:
    return re.sub(r"[^a-z0-9]", "", k.lower())


def _rows(path):
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            yield {_norm(k): v for k, v in r.items() if k is not None}


def _find(dirpath, suffix):
    hits = sorted(glob.glob(os.path.join(dirpath, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {dirpath}")
    return hits


def kernel_durations(trace_dir, kernel_regex):
    """(start, duration ns) of every dispatch of the kernel, in launch order."""
    rx = re.compile(kernel_regex)
    out = []
    for path in _find(trace_dir, "kernel_trace.csv"):
        for r in _rows(path):
            if rx.search(r.get("kernelname", "")):
                s, e = int(r["starttimestamp"]), int(r["endtimestamp"])
                out.append((s, e - s))
    out.sort()
    return [d for _, d in out]


def counter_values(pmc_dir, kernel_regex):
    """{counter: [per-dispatch value, in launch order]} for the kernel's dispatches."""
    rx = re.compile(kernel_regex)
    per = {}  # (order key, counter) -> value
    for path in _find(pmc_dir, "counter_collection.csv"):
        for r in _rows(path):
            if not rx.search(r.get("kernelname", "")):
                continue
            key = int(r.get("dispatchid") or r.get("correlationid") or 0)
            name = r["countername"]
            per[(key, name)] = per.get((key, name), 0.0) + float(r["countervalue"])
    out = {}
    for (key, name), v in sorted(per.items()):
        out.setdefault(name, []).append(v)
    return out


def summarize(name, kernel_regex, flops, compulsory, trace_dir, pmc_dirs, skip, peak=PEAK_BF16_TFLOPS):
    d = kernel_durations(trace_dir, kernel_regex)
    if len(d) <= skip:
        raise ValueError(f"{len(d)} dispatches of {kernel_regex!r}, fewer than --skip {skip} + 1")
    timed = d[skip:]
    rec = {"dispatches": len(d), "timed": len(timed), "avg_ns_timed": statistics.fmean(timed),
           "median_ns_timed": statistics.median(timed), "min_ns_timed": min(timed), "max_ns_timed": max(timed),
           "avg_ns_all": statistics.fmean(d), "max_ns_all": max(d)}
    rec["achieved_tflops"] = flops / (rec["avg_ns_timed"] * 1e-9) / 1e12
    rec["frac"] = rec["achieved_tflops"] / peak
    counters = {}
    for pd in pmc_dirs:
        for cname, vals in counter_values(pd, kernel_regex).items():
            v = vals[skip:] if len(vals) > skip else vals
            counters[cname] = statistics.fmean(v)
    rec["counters"] = counters
    if "FETCH_SIZE" in counters and "WRITE_SIZE" in counters:
        rb = counters["FETCH_SIZE"] * 1024 * FETCH_FACTOR
        wb = counters["WRITE_SIZE"] * 1024 * WRITE_FACTOR
        rec.update(read_bytes=rb, write_bytes=wb, hbm_bytes=rb + wb, compulsory_bytes=compulsory,
                   traffic_ratio=(rb + wb) / compulsory)
    if "GRBM_GUI_ACTIVE" in counters:
        cyc = counters["GRBM_GUI_ACTIVE"] / NUM_XCD
        rec["cycles"] = cyc
        rec["sclk_ghz"] = cyc / rec["avg_ns_timed"]
        if "SQ_VALU_MFMA_BUSY_CYCLES" in counters:
            rec["mfma_busy"] = counters["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * NUM_SIMD)
        if "SQ_ACTIVE_INST_VALU" in counters:
            rec["valu_busy"] = 4 * counters["SQ_ACTIVE_INST_VALU"] / NUM_SIMD / cyc
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in counters:
            rec["coexec"] = counters["SQ_VALU_MFMA_COEXEC_CYCLES"] / (cyc * NUM_SIMD)
        if "SQ_LDS_BANK_CONFLICT" in counters:
            rec["lds_conflict"] = counters["SQ_LDS_BANK_CONFLICT"] / NUM_CU / cyc
    return rec


def markdown(name, workload_desc, rec, cmds, skip, source_hash, peak=PEAK_BF16_TFLOPS, peak_label="bf16"):
    L = [f"# {name} on {workload_desc}", "",
         f"Kernel source hash (`kernel_source_hash`): `{source_hash}`. Commands (run from the repository root):", ""]
    L += ["    " + c for c in cmds]
    L += ["", "## Kernel trace (`--kernel-trace --stats`)", "",
          f"{rec['dispatches']} dispatches of the kernel; the first {skip} are the command's warm-up launches and are "
          f"left out, the other {rec['timed']} are the timed launches.", "",
          "| dispatches | average (ns) | median (ns) | min (ns) | max (ns) |", "|---|---|---|---|---|",
          f"| timed ({rec['timed']}) | {rec['avg_ns_timed']:.0f} | {rec['median_ns_timed']:.0f} | {rec['min_ns_timed']} | "
          f"{rec['max_ns_timed']} |",
          f"| all ({rec['dispatches']}) | {rec['avg_ns_all']:.0f} | | | {rec['max_ns_all']} |", "",
          f"Algorithmic work per launch / timed average duration = {rec['achieved_tflops']:.1f} TFLOP/s = "
          f"{100 * rec['frac']:.1f}% of the {peak:.0f} TFLOP/s dense {peak_label} peak."]
    if "hbm_bytes" in rec:
        c = rec["counters"]
        L += ["", "## HBM traffic (per timed launch, calibrated by a 1 GiB device copy)", "",
              "| | KiB (counter) | bytes (calibrated) |", "|---|---|---|",
              f"| FETCH_SIZE | {c['FETCH_SIZE']:.0f} | {rec['read_bytes']:.4e} |",
              f"| WRITE_SIZE | {c['WRITE_SIZE']:.0f} | {rec['write_bytes']:.4e} |",
              f"| total | | {rec['hbm_bytes']:.4e} |",
              f"| compulsory Q+K+V read, O+LSE written | | {rec['compulsory_bytes']:.4e} |", "",
              f"Traffic / compulsory = {rec['traffic_ratio']:.2f}; at the timed duration that is "
              f"{rec['hbm_bytes'] / rec['avg_ns_timed']:.0f} GB/s of HBM traffic (peak {PEAK_HBM_GBPS:.0f} GB/s)."]
    sq = {k: v for k, v in rec["counters"].items() if k not in ("FETCH_SIZE", "WRITE_SIZE")}
    if sq:
        L += ["", "## SQ counters (per timed dispatch)", "", "| counter | value |", "|---|---|"]
        L += [f"| {k} | {v:.4e} |" for k, v in sorted(sq.items())]
        if "cycles" in rec:
            L += ["", f"Derived ({NUM_XCD} XCDs, {NUM_CU} CUs, {NUM_SIMD} SIMDs; GRBM_GUI_ACTIVE summed over XCDs; "
                  "SQ_ACTIVE_INST_VALU in units of 4 cycles):", "",
                  f"* kernel cycles per XCD {rec['cycles']:.4e}: effective shader clock {rec['sclk_ghz']:.2f} GHz"]
            for key, label in (("mfma_busy", "MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES / cycles / SIMDs)"),
                               ("valu_busy", "VALU busy"), ("coexec", "MFMA and VALU co-executing"),
                               ("lds_conflict", "LDS bank-conflict cycles per CU")):
                if key in rec:
                    L.append(f"* {label} = {100 * rec[key]:.1f}%")
    return "\n".join(L) + "\n"


def launch_table(trace_dir, pmc_dirs, specs, skip):
    """Rows for launch groups of several kernels in one run. specs: (label, regex, count) in
    launch order; the k-th group of a regex takes that regex's next `count` dispatches (in launch
    order), and the first `skip` of each group are left out (warm-ups)."""
    disp = []
    for path in _find(trace_dir, "kernel_trace.csv"):
        for r in _rows(path):
            disp.append((int(r["starttimestamp"]), r["kernelname"], int(r["endtimestamp"]) - int(r["starttimestamp"])))
    disp.sort()
    counters = {}  # counter -> [(dispatch id, kernel name, value)] in launch order
    for pd in pmc_dirs:
        for path in _find(pd, "counter_collection.csv"):
            per = {}
            for r in _rows(path):
                key = (int(r.get("dispatchid") or r.get("correlationid") or 0), r["kernelname"], r["countername"])
                per[key] = per.get(key, 0.0) + float(r["countervalue"])
            for (did, kname, cname), v in sorted(per.items()):
                counters.setdefault(cname, []).append((kname, v))
    cursor = {}
    out = []
    for label, regex, count in specs:
        rx = re.compile(regex)
        mine = [(n, d) for _, n, d in disp if rx.search(n)]
        c0 = cursor.get(regex, 0)
        cursor[regex] = c0 + count
        timed = list(range(c0 + skip, c0 + count))
        if not timed or timed[-1] >= len(mine):
            raise ValueError(f"{label}: {len(mine)} dispatches of {regex!r}, group {c0}..{c0 + count - 1} missing")
        row = {"label": label, "kernel": mine[c0][0], "launches": len(timed),
               "mean_ms": statistics.fmean(mine[i][1] for i in timed) / 1e6}
        for cname, factor in (("FETCH_SIZE", FETCH_FACTOR), ("WRITE_SIZE", WRITE_FACTOR)):
            series = [v for kname, v in counters.get(cname, []) if rx.search(kname)]
            if len(series) > timed[-1]:
                row[cname] = statistics.fmean(series[i] for i in timed) * 1024 * factor
        out.append(row)
    return out


def launches_markdown(title, rows, cmds, skip, source_hash):
    L = [f"# {title}", "", f"Kernel source hash (`kernel_source_hash`): `{source_hash}`. Commands (run from the "
         "repository root):", ""]
    L += ["    " + c for c in cmds]
    L += ["", f"Per launch group, the first {skip} launches (warm-ups) are left out. Fetched / written = "
          f"{FETCH_FACTOR:.1f} x FETCH_SIZE, {WRITE_FACTOR:.1f} x WRITE_SIZE (KiB, copy calibration): the L2's traffic "
          "to the memory fabric.", "",
          "| launch | kernel | launches | mean (ms) | fetched (GB) | written (GB) | GB/s |", "|---|---|---|---|---|---|---|"]
    for r in rows:
        fb, wb = r.get("FETCH_SIZE"), r.get("WRITE_SIZE")
        gbs = (fb + wb) / (r["mean_ms"] * 1e6) if fb is not None and wb is not None else None
        kn = re.sub(r"^void |\(fa::FwdParams\)$", "", r["kernel"])
        L.append(f"| {r['label']} | `{kn}` | {r['launches']} | {r['mean_ms']:.3f} | "
                 f"{'' if fb is None else f'{fb / 1e9:.2f}'} | {'' if wb is None else f'{wb / 1e9:.3f}'} | "
                 f"{'' if gbs is None else f'{gbs:.0f}'} |")
    return "\n".join(L) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--launch", action="append", default=[],
                    help="LABEL=REGEX=COUNT, in launch order: a table of launch groups instead of one kernel")
    ap.add_argument("--title", default="")
    ap.add_argument("--name")
    ap.add_argument("--kernel-regex")
    ap.add_argument("--workload")
    ap.add_argument("--causal", action="store_true")
    ap.add_argument("--skip", type=int, default=5)
    ap.add_argument("--trace", required=True)
    ap.add_argument("--pmc", action="append", default=[])
    ap.add_argument("--cmd", action="append", default=[])
    ap.add_argument("--out", required=True)
    ap.add_argument("--traffic-json")
    ap.add_argument("--peak-tflops", type=float, default=PEAK_BF16_TFLOPS,
                    help="dense MFMA peak the kernel is priced against (fp8: 5000)")
    ap.add_argument("--peak-label", default="bf16")
    a = ap.parse_args(argv)
    if a.launch:
        specs = []
        for spec in a.launch:
            label, regex, count = spec.rsplit("=", 2)
            specs.append((label, regex, int(count)))
        rows = launch_table(a.trace, a.pmc, specs, a.skip)
        with open(a.out, "w") as f:
            f.write(launches_markdown(a.title, rows, a.cmd, a.skip, kernel_source_hash()))
        print(json.dumps(rows))
        return
    sys.path.insert(0, ROOT)
    from exact_attention_06_amd import workloads as W

    w = W.by_name(a.workload)
    flops = w.flops(a.causal)
    compulsory = 2 * w.B * w.d * (2 * w.N * w.Hq + 2 * w.N * w.Hkv) + 4 * w.B * w.Hq * w.N
    rec = summarize(a.name, a.kernel_regex, flops, compulsory, a.trace, a.pmc, a.skip, a.peak_tflops)
    h = kernel_source_hash()
    desc = (f"{w.name} (B={w.B}, N={w.N}, Hq={w.Hq}, Hkv={w.Hkv}, d={w.d}, "
            f"{'causal' if a.causal else 'non-causal'})")
    with open(a.out, "w") as f:
        f.write(markdown(a.name, desc, rec, a.cmd, a.skip, h, a.peak_tflops, a.peak_label))
    if a.traffic_json:
        db = json.load(open(a.traffic_json)) if os.path.exists(a.traffic_json) else {}
        e = {"workload": w.name, "causal": a.causal, "source_hash": h, "timed_dispatches": rec["timed"],
             "avg_launch_ns": round(rec["avg_ns_timed"]), "achieved_tflops": round(rec["achieved_tflops"], 1),
             "frac": round(rec["frac"], 4)}
        if "hbm_bytes" in rec:
            e.update(hbm_bytes_per_launch=round(rec["hbm_bytes"]), read_bytes=round(rec["read_bytes"]),
                     write_bytes=round(rec["write_bytes"]), compulsory_bytes=rec["compulsory_bytes"],
                     fetch_size_kib=rec["counters"]["FETCH_SIZE"], write_size_kib=rec["counters"]["WRITE_SIZE"],
                     fetch_factor=FETCH_FACTOR, write_factor=WRITE_FACTOR)
        for k in ("sclk_ghz", "mfma_busy", "valu_busy", "coexec"):
            if k in rec:
                e[k] = round(rec[k], 4)
        db[a.name] = e
        with open(a.traffic_json, "w") as f:
            json.dump(db, f, indent=1)
    print(json.dumps({k: v for k, v in rec.items() if k != "counters"}))


if __name__ == "__main__":
    main()
