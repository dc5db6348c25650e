"""Per-case parity figures of the GPU tests, kept as a record (test infrastructure only).

When the environment variable FA_PARITY_RECORD names a file, every bf16/fp16 forward
comparison appends one JSON line to it: the case, O max-abs (all elements and those with
|O_ref| < 4), O mean-abs, LSE max-abs, the number of sampled elements with |O_ref| >= 4 and
their worst error in excess of half a bf16 ulp of O_ref (the spiked stress case also gives how
many elements with |O_ref| < 4 land above 1e-2). Run as a script it turns such a file into a
markdown table:

    python tests/parity_record.py RECORD.jsonl > profiles/parity_record.md
"""

import json
import os
import re
import sys

O_MAX = 1e-2


def record(**entry):
    path = os.environ.get("FA_PARITY_RECORD")
    if not path:
        return
    with open(path, "a") as f:
        f.write(json.dumps(entry) + "\n")


# the workloads the benchmark and the pages' configurations name (tiny, ragged, the hd128 /
# hd256 / hd512 sweeps, the spiked-key video shape): listed case by case
NAMED = re.compile(r"^(tiny|ragged|hd128_N\d+_(mha|gqa4)|hd256_N\d+|hd512_N\d+|video)(/|$)")


def _line(r):
    flag = r["o_max"] > O_MAX and r["o_max_small"] <= O_MAX
    ex = f"{r['ex_big']:.2e}" if r["n_big"] else "-"
    return (f"| {r['case']} | {r['o_max']:.2e} | {r['o_max_small']:.2e} | {r['o_mean']:.2e} | {r['lse_max']:.2e} "
            f"| {r['n_big']} | {ex} | {'yes' if flag else 'no'} |")


HEADER = """# Parity record: every bf16/fp16 forward comparison of the GPU suite

One GPU run of the whole suite on the current kernel sources, each case against the fp64 oracle (all rows, or the
seeded sampled rows of the full-size workloads). Commands (from the repository root):

    FA_PARITY_RECORD=gpurun_out/parity.jsonl python -u -m pytest tests -m gpu -x -v -s
    python3 tests/parity_record.py gpurun_out/parity.jsonl > profiles/parity_record.md

The bar: O max-abs <= 1e-2 and mean-abs <= 1e-3, LSE max-abs <= 1e-3. Where |O_ref| >= 4 the bf16 grid spacing is
2^-5, so the correctly rounded value itself can be 1.56e-2 away; such elements are held to half a bf16 ulp plus
1e-2 - 2^-7, and the tables give their count and worst excess over the half ulp. One stress case (spiked keys, 9.4M
compared elements) is held instead to at most one element in a million with |O_ref| < 4 above 1e-2 and none above
1.1e-2: P enters the P.V product in bf16, and on rows dominated by a few keys its rounding can carry such an element
just past the bar. A case that two tests check with the same figures is listed once.
"""


def main(path):
    rows, seen = [], set()
    for line in open(path):
        if line.strip() and line.strip() not in seen:
            seen.add(line.strip())
            rows.append(json.loads(line))
    print(HEADER)
    named = [r for r in rows if NAMED.match(r["case"])]
    other = [r for r in rows if not NAMED.match(r["case"])]
    head = ("| case | O max-abs | O max-abs, \\|O_ref\\| < 4 | O mean-abs | LSE max-abs | elements with \\|O_ref\\| >= 4 "
            "| their worst excess over half a bf16 ulp | over 1e-2 only on \\|O_ref\\| >= 4 |")
    print("## Named workloads (configurations and sweeps)")
    print()
    print(head)
    print("|---|---|---|---|---|---|---|---|")
    for r in named:
        print(_line(r))
    print()
    print("## Every other case (small, ragged, rectangular, GQA, zero / negative / large scales, split-KV, random")
    print("shapes, variable-length and paged), summarised")
    print()
    if other:
        print(f"{len(other)} cases: largest O max-abs {max(r['o_max'] for r in other):.3e}, largest O max-abs on "
              f"|O_ref| < 4 {max(r['o_max_small'] for r in other):.3e}, largest O mean-abs "
              f"{max(r['o_mean'] for r in other):.3e}, largest LSE max-abs {max(r['lse_max'] for r in other):.3e}, "
              f"{sum(r['n_big'] for r in other)} elements with |O_ref| >= 4.")
        big = [r for r in other if r["o_max"] > O_MAX]
        if big:
            print()
            print("Cases above 1e-2 (on |O_ref| >= 4 elements only where the last column says so):")
            print()
            print(head)
            print("|---|---|---|---|---|---|---|---|")
            for r in big:
                print(_line(r))
    tail = [r for r in rows if "n_over" in r]
    if tail:
        print()
        print("## Stress case with the bf16-P tail allowance (elements with |O_ref| < 4 above 1e-2)")
        print()
        print("| case | elements compared | above 1e-2 with \\|O_ref\\| < 4 | their largest error | O mean-abs | LSE max-abs |")
        print("|---|---|---|---|---|---|")
        for r in tail:
            print(f"| {r['case']} | {r['n_elems']} | {r['n_over']} | {r['o_max_small']:.3e} | {r['o_mean']:.2e} "
                  f"| {r['lse_max']:.2e} |")
    print()
    only_big = [r["case"] for r in rows if r["o_max"] > O_MAX and r["o_max_small"] <= O_MAX]
    worst = max(rows, key=lambda r: r["o_max"])
    print(f"All {len(rows)} cases: largest O max-abs {worst['o_max']:.3e} ({worst['case']}), largest LSE max-abs "
          f"{max(r['lse_max'] for r in rows):.3e}, largest O mean-abs {max(r['o_mean'] for r in rows):.3e}; "
          f"largest O max-abs on |O_ref| < 4 {max(r['o_max_small'] for r in rows):.3e}.")
    if only_big:
        print(f"Above 1e-2 only on elements with |O_ref| >= 4: {', '.join(sorted(set(only_big)))}.")
    small_over = sorted({r["case"] for r in rows if r["o_max_small"] > O_MAX})
    if small_over:
        print(f"Above 1e-2 on elements with |O_ref| < 4: {', '.join(small_over)} (the stress case above).")
    elif not only_big:
        print("No case exceeds 1e-2 on any element.")


if __name__ == "__main__":
    main(sys.argv[1])
