"""The rocprofv3 summarizer on synthetic CSV files (CPU only): warm-up dispatches are left
out, only the named kernel counts, counters are averaged per timed dispatch and the HBM bytes
follow the copy calibration."""

import json
import os

from exact_attention_06_amd import profile_summary as P
from exact_attention_06_amd import workloads as W

K = "void fa::fwd_kernel<256, false, fa::Bf16, 0, 4>(fa::FwdParams)"
OTHER = "void fa::fwd_combine<256, fa::Bf16>(fa::FwdParams)"


def _trace(d, durations):
    os.makedirs(d)
    with open(os.path.join(d, "run_kernel_trace.csv"), "w") as f:
        f.write('"Kind","Dispatch_Id","Kernel_Name","Start_Timestamp","End_Timestamp"\n')
        t = 1000
        for i, dur in enumerate(durations):
            f.write(f'"KERNEL_DISPATCH",{2 * i},"{K}",{t},{t + dur}\n')
            f.write(f'"KERNEL_DISPATCH",{2 * i + 1},"{OTHER}",{t + dur},{t + dur + 5}\n')
            t += dur + 100


def _pmc(d, counter, values):
    os.makedirs(d)
    with open(os.path.join(d, "run_counter_collection.csv"), "w") as f:
        f.write('"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value"\n')
        for i, v in enumerate(values):
            f.write(f'{2 * i},"{K}","{counter}",{v}\n')
            f.write(f'{2 * i + 1},"{OTHER}","{counter}",999999\n')


def test_summary_skips_warmup_and_other_kernels(tmp_path):
    durations = [5000, 4000, 3000, 1000, 1000, 1000]     # two warm-ups, then four timed launches
    _trace(str(tmp_path / "tr"), durations)
    _pmc(str(tmp_path / "f"), "FETCH_SIZE", [7, 7, 100, 100, 100, 100])
    _pmc(str(tmp_path / "w"), "WRITE_SIZE", [7, 7, 50, 50, 50, 50])
    rec = P.summarize("k", r"fwd_kernel<256, false", 2.0e12, 1.0e6, str(tmp_path / "tr"),
                      [str(tmp_path / "f"), str(tmp_path / "w")], skip=2)
    assert rec["dispatches"] == 6 and rec["timed"] == 4
    assert rec["avg_ns_timed"] == 1500.0 and rec["max_ns_timed"] == 3000
    assert abs(rec["achieved_tflops"] - 2.0e12 / 1500e-9 / 1e12) < 1e-6
    assert rec["counters"]["FETCH_SIZE"] == 100 and rec["counters"]["WRITE_SIZE"] == 50
    assert rec["hbm_bytes"] == 100 * 1024 * 2.0 + 50 * 1024 * 1.0


def test_main_writes_markdown_and_traffic_json(tmp_path):
    _trace(str(tmp_path / "tr"), [9000] * 5 + [1000] * 20)
    out, tj = str(tmp_path / "s.md"), str(tmp_path / "t.json")
    P.main(["--name", "fwd_kernel<256,noncausal,bf16>", "--kernel-regex", r"fwd_kernel<256, false",
            "--workload", "hd256_N8192", "--skip", "5", "--trace", str(tmp_path / "tr"), "--cmd", "x", "--out", out,
            "--traffic-json", tj])
    text = open(out).read()
    assert "timed (20) | 1000 |" in text
    e = json.load(open(tj))["fwd_kernel<256,noncausal,bf16>"]
    w = W.by_name("hd256_N8192")
    assert e["avg_launch_ns"] == 1000 and abs(e["achieved_tflops"] - w.flops(False) / 1e-6 / 1e12) < 0.1
    assert e["source_hash"] == P.kernel_source_hash()


def test_launch_table_groups_by_regex_in_launch_order(tmp_path):
    # two groups of 3 launches of K (warm-up 1 each), OTHER interleaved with the second group
    d = tmp_path / "tr"
    os.makedirs(d)
    rows, t, i = [], 1000, 0
    for k, dur in [(K, 900), (K, 100), (K, 100), (K, 900), (OTHER, 7), (K, 300), (OTHER, 9), (K, 300), (OTHER, 11)]:
        rows.append(f'"KERNEL_DISPATCH",{i},"{k}",{t},{t + dur}\n')
        t += dur + 50
        i += 1
    with open(d / "run_kernel_trace.csv", "w") as f:
        f.write('"Kind","Dispatch_Id","Kernel_Name","Start_Timestamp","End_Timestamp"\n' + "".join(rows))
    os.makedirs(tmp_path / "f")
    with open(tmp_path / "f" / "run_counter_collection.csv", "w") as f:
        f.write('"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value"\n')
        for j, (k, v) in enumerate([(K, 1), (K, 10), (K, 10), (K, 1), (OTHER, 2), (K, 20), (OTHER, 4), (K, 20),
                                    (OTHER, 6)]):
            f.write(f'{j},"{k}","FETCH_SIZE",{v}\n')
    specs = [("a", r"fwd_kernel<256", 3), ("b", r"fwd_kernel<256", 3), ("m", r"fwd_combine", 3)]
    out = P.launch_table(str(d), [str(tmp_path / "f")], specs, skip=1)
    assert [r["launches"] for r in out] == [2, 2, 2]
    assert [r["mean_ms"] for r in out] == [100 / 1e6, 300 / 1e6, 10 / 1e6]
    assert [r["FETCH_SIZE"] for r in out] == [10 * 1024 * P.FETCH_FACTOR, 20 * 1024 * P.FETCH_FACTOR,
                                              5 * 1024 * P.FETCH_FACTOR]
    assert "WRITE_SIZE" not in out[0]
    md = P.launches_markdown("t", out, ["c"], 1, "h")
    assert md.count("\n| ") == 4 and "| b | `fa::fwd_kernel<256, false, fa::Bf16, 0, 4>` | 2 | 0.000 |" in md
