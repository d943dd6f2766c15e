"""Turn the parity records of the benchmark configurations into a markdown report.

Usage: python -m tests.parity_report [RECORD_DIR] [OUT.md]

Reads RECORD_DIR/report_<workload>.json (written by
tests/test_gpu_parity_report.py on the GPU; RECORD_DIR defaults to the
records folder of tests/parity.py) and prints, or writes, a table
per configuration plus the records themselves as one JSON block at the end.
CPU only; it reads the JSON records and calls nothing else.
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORDER = ["tiny", "distilbert", "bf16_l512", "long_l8192", "layer_bf16"]


def parity_records_dir():
    from tests import parity
    return parity.RECORD_DIR


def load(record_dir):
    recs = {}
    for name in ORDER:
        path = os.path.join(record_dir, f"report_{name}.json")
        if os.path.exists(path):
            with open(path) as f:
                recs[name] = json.load(f)
    return recs


def render(recs) -> str:
    lines = ["| workload | plan | tokens | near-ties (per iteration) | excused flips | "
             "bad | zero-centroid tokens (last iteration) | free-running mismatches | "
             "max dist err / ||q||^2 | max abs(out - oracle) (tol) |",
             "|---|---|---|---|---|---|---|---|---|---|"]
    for name in ORDER:
        r = recs.get(name)
        if r is None:
            lines.append(f"| {name} | (no record) | | | | | | | | |")
            continue
        its = r["iterations"]
        toks = r["B"] * r["H"] * r["L"]
        lines.append(
            f"| {name} | {r['plan']} | {toks} | "
            + ", ".join(str(i["near_ties"]) for i in its)
            + f" | {r['excused']} | {r['bad']} | {r['zero_centroid_tokens_last']} | "
            f"{r['free_running_mismatches']} | {r['max_dist_err_rel']:.2e} | "
            f"{r['max_out_err']:.2e} ({r['tol']}) |")
    return "\n".join(lines)


def main():
    record_dir = sys.argv[1] if len(sys.argv) > 1 else parity_records_dir()
    recs = load(record_dir)
    text = render(recs) + "\n\n```json\n" + json.dumps(recs, indent=1, sort_keys=True) + "\n```\n"
    if len(sys.argv) > 2:
        with open(sys.argv[2], "w") as f:
            f.write(text)
    else:
        print(text)


if __name__ == "__main__":
    main()
