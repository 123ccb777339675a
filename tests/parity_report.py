"""Summarises the per-case parity reports that the GPU tests append to the file DG_PARITY_LOG
names (one JSON object per comparison) as a markdown table: per test, the compared rows, the
exempt rows of each kind and how many of them differ, and the largest statistic errors.

    DG_PARITY_LOG=gpurun_out/parity.jsonl python -m pytest tests -m gpu
    python tests/parity_report.py gpurun_out/parity.jsonl > profiles/parity_counts.md
"""
import collections
import json
import sys


def main(path: str) -> int:
    agg = collections.OrderedDict()
    keys_sum = ("rows", "commit_rows", "argmax_exempt", "argmax_exempt_differ", "gumbel_exempt",
                "gumbel_exempt_differ", "accept_exempt", "accept_exempt_differ", "conv_exempt")
    keys_max = ("lse_max_rel", "entropy_max_rel", "sc_max_rel", "margin_max")
    n = 0
    with open(path) as f:
        for line in f:
            rec = json.loads(line)
            n += 1
            a = agg.setdefault(rec.get("test", "?"), {"cases": 0})
            a["cases"] += 1
            for k in keys_sum:
                if k in rec:
                    a[k] = a.get(k, 0) + int(rec[k])
            for k in keys_max:
                if k in rec:
                    a[k] = max(a.get(k, 0.0), float(rec[k]))
    print("# Parity counts of a GPU test run")
    print()
    print("Commands (repository root, on the GPU):")
    print()
    print("    DG_PARITY_LOG=gpurun_out/parity.jsonl python -m pytest tests -m gpu")
    print("    python tests/parity_report.py gpurun_out/parity.jsonl > profiles/parity_counts.md")
    print()
    print("Per test (summed over its comparisons): rows compared, rows of committing canvases,")
    print("exempt decisions (oracle margin below the limit) and how many of those differ, and")
    print("the largest relative errors of the statistics and the expectation. Any difference")
    print("outside an exemption fails its test, so none appears here.")
    print()
    print(f"Comparisons: {n}, tests: {len(agg)}.")
    print()
    cols = ("cases",) + keys_sum + keys_max
    print("| test | " + " | ".join(cols) + " |")
    print("|---|" + "---|" * len(cols))
    tot = collections.Counter()
    for t, a in agg.items():
        cells = []
        for k in cols:
            v = a.get(k)
            if v is None:
                cells.append("")
            elif isinstance(v, float):
                cells.append(f"{v:.2e}")
            else:
                cells.append(str(v))
                tot[k] += v
        print(f"| {t.split('::', 1)[-1] if '::' in t else t} ({t.split('::')[0].split('/')[-1]}) | "
              + " | ".join(cells) + " |")
    print("| **total** | " + " | ".join(str(tot[k]) if k in tot else "" for k in cols) + " |")
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1]))
