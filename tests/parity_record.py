"""Per-case parity figures of the GPU tests, kept as a record (test infrastructure only).

When the environment variable FA_PARITY_RECORD names a file, every bf16/fp16 forward
comparison appends one JSON line to it: the case, O max-abs (all elements and those with
|O_ref| < 4), O mean-abs, LSE max-abs, the number of sampled elements with |O_ref| >= 4 and
their worst error in excess of half a bf16 ulp of O_ref. Run as a script it turns such a file
into a markdown table:

    python tests/parity_record.py RECORD.jsonl > profiles/parity_record.md
"""

import json
import os
import sys

O_MAX = 1e-2


def record(**entry):
    path = os.environ.get("FA_PARITY_RECORD")
    if not path:
        return
    with open(path, "a") as f:
        f.write(json.dumps(entry) + "\n")


def main(path):
    rows = [json.loads(line) for line in open(path) if line.strip()]
    print("| case | O max-abs | O max-abs, \\|O_ref\\| < 4 | O mean-abs | LSE max-abs | elements with \\|O_ref\\| >= 4 "
          "| their worst excess over half a bf16 ulp | over 1e-2 only on \\|O_ref\\| >= 4 |")
    print("|---|---|---|---|---|---|---|---|")
    only_big = []
    for r in rows:
        flag = r["o_max"] > O_MAX and r["o_max_small"] <= O_MAX
        if flag:
            only_big.append(r["case"])
        ex = f"{r['ex_big']:.2e}" if r["n_big"] else "-"
        print(f"| {r['case']} | {r['o_max']:.2e} | {r['o_max_small']:.2e} | {r['o_mean']:.2e} | {r['lse_max']:.2e} "
              f"| {r['n_big']} | {ex} | {'yes' if flag else 'no'} |")
    print()
    worst = max(rows, key=lambda r: r["o_max"]) if rows else None
    print(f"{len(rows)} cases. Largest O max-abs: {worst['o_max']:.3e} ({worst['case']}). "
          f"Largest LSE max-abs: {max(r['lse_max'] for r in rows):.3e}. Largest O mean-abs: "
          f"{max(r['o_mean'] for r in rows):.3e}.")
    if only_big:
        print(f"Cases above 1e-2 only on elements with |O_ref| >= 4: {', '.join(only_big)}.")
    else:
        print("No case exceeds 1e-2 on any element, including those with |O_ref| >= 4.")


if __name__ == "__main__":
    main(sys.argv[1])
