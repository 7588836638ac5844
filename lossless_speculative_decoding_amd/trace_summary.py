"""Summarise a rocprofv3 kernel trace of one bench.py run.

Input: the directory rocprofv3 wrote (``--kernel-trace --output-format csv -d DIR``) and the
log of that same bench.py run (its last line is the JSON record).  Output (markdown):

- the whole run's kernels by total time (calls, average and total duration, share);
- the metric kernel's dispatches that bench.py counted as warmup and timed: bench.py reports
  how many launches of the draft-attention class it timed (``roofline.launches``) and how many
  it made up to the end of the timed region (``launches_incl_warmup``); those are the first
  ``launches_incl_warmup`` dispatches of the kernel in dispatch order, the last ``launches`` of
  them timed.  Their average rocprofv3 duration and the algorithmic bytes per launch give the
  profiler's view of the roofline figure, beside bench.py's live one.

    python -m lossless_speculative_decoding_amd.trace_summary DIR bench.log [--kernel attn_decode_bf16]
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import json


def short_name(name: str) -> str:
    """The kernel's name without namespaces, return type and argument list (template arguments
    kept); library kernels from other projects cut to 90 characters."""
    n = name.replace("(anonymous namespace)::", "")
    if n.startswith("void "):
        n = n[5:]
    depth = 0
    for i, ch in enumerate(n):
        depth += ch == "<"
        depth -= ch == ">"
        if ch == "(" and depth == 0:
            n = n[:i]
            break
    return n.replace("vc::", "")[:90]


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("trace_dir")
    ap.add_argument("bench_log")
    ap.add_argument("--kernel", default="attn_decode_bf16")
    ap.add_argument("--top", type=int, default=12)
    a = ap.parse_args()
    rec = json.loads([ln for ln in open(a.bench_log) if ln.startswith("{")][-1])
    rf = rec["roofline"]
    rows = []
    for f in glob.glob(f"{a.trace_dir}/**/*kernel_trace.csv", recursive=True):
        for r in csv.DictReader(open(f)):
            rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    if not rows:
        raise SystemExit(f"no kernel_trace.csv under {a.trace_dir}")
    rows.sort()
    tot = collections.defaultdict(lambda: [0, 0])
    for _, name, dur in rows:
        t = tot[short_name(name)]
        t[0] += 1
        t[1] += dur
    all_ns = sum(v[1] for v in tot.values())
    print("| kernel | calls | avg us | total ms | % |\n|---|---|---|---|---|")
    for name, (c, t) in sorted(tot.items(), key=lambda kv: -kv[1][1])[: a.top]:
        print(f"| `{name}` | {c} | {t / c / 1e3:.2f} | {t / 1e6:.1f} | {100 * t / all_ns:.1f} |")
    mine = [dur for _, name, dur in rows if a.kernel in name]
    n_all, n_timed = rf["launches_incl_warmup"], rf["launches"]
    timed = mine[n_all - n_timed:n_all]
    if len(timed) != n_timed:
        raise SystemExit(f"{len(mine)} dispatches of {a.kernel} in the trace, fewer than bench.py's {n_all}")
    avg_us = sum(timed) / len(timed) / 1e3
    bpl = rf["bytes_per_launch"]
    gbs = bpl / avg_us / 1e3
    print()
    print(f"`{a.kernel}`: {len(mine)} dispatches in the trace; bench.py counted {n_all} up to the end of its timed "
          f"region, the last {n_timed} timed.")
    print(f"Timed region: rocprofv3 average {avg_us:.2f} us per launch, {bpl / 1e6:.1f} MB algorithmic per launch "
          f"-> {gbs:.0f} GB/s = {gbs / 8000 * 100:.1f}% of 8 TB/s; bench.py live in the same run "
          f"{rf['avg_launch_ms'] * 1e3:.2f} us ({rf['achieved']} GB/s = {rf['frac'] * 100:.1f}%); "
          f"{rec['scheduler'].get('mean_requests_per_draft_step')} requests per draft step.")


if __name__ == "__main__":
    main()
