"""Summarise rocprofv3 HBM byte counters of one kernel into a profile record.

Two counter passes of the measured command (FETCH_SIZE, then WRITE_SIZE, KiB per
dispatch) and the same two passes over a plain copy kernel of known size
(``bench.py --calibrate-copy``: 1 GiB read, 1 GiB written per dispatch) give
HBM bytes per dispatch: each counter's average over the kernel's dispatches,
times (known copy bytes / what that counter read for the copy).  The record
keeps a hash of the kernel's source files; bench.py reports the traffic only
while those files are unchanged.

    python -m lossless_speculative_decoding_amd.pmc_summary --kernel attn_decode_bf16 \\
        --fetch F.csv --write W.csv --copy-fetch CF.csv --copy-write CW.csv \\
        --command "..." --out profiles/NAME.json
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os

HERE = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 1 << 30
COPY_KERNEL = "direct_copy_kernel"
# sources that define each profiled kernel and its launch
KERNEL_SOURCES = {
    "attn_decode_bf16": ["csrc/attention.hip", "csrc/attention.h", "csrc/common.h"],
    "attn_quant": ["csrc/attention_quant.hip", "csrc/attention_quant.h", "csrc/attention.h", "csrc/common.h"],
    "attn_rows_bf16": ["csrc/attention_rows.hip", "csrc/attention.h", "csrc/common.h"],
}


def sources_sha256(kernel: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()


def counter_avg(path: str, kernel: str, counter: str, first: int | None = None,
                last: int | None = None) -> tuple[float, int]:
    """Average of the counter over the dispatches of kernels whose name contains `kernel` (the
    first `first` or the last `last` of them in dispatch order when given)."""
    rows = sorted((r for r in csv.DictReader(open(path)) if kernel in r["Kernel_Name"] and r["Counter_Name"] == counter),
                  key=lambda r: int(r["Dispatch_Id"]))
    if last is not None:
        rows = rows[-last:]
    vals = [float(r["Counter_Value"]) for r in rows[:first]]
    if not vals:
        raise SystemExit(f"no {counter} rows for a kernel named like {kernel!r} in {path}")
    return sum(vals) / len(vals), len(vals)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--kernel", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-fetch", required=True)
    ap.add_argument("--copy-write", required=True)
    ap.add_argument("--algorithmic-bytes", type=float, default=None,
                    help="algorithmic bytes per dispatch over the same dispatches, for the ratio")
    ap.add_argument("--first", type=int, default=None,
                    help="only the kernel's first N dispatches (those the algorithmic bytes describe)")
    ap.add_argument("--last", type=int, default=None,
                    help="only the kernel's last N dispatches (e.g. a timed region followed by no other "
                         "dispatch of the same kernel)")
    ap.add_argument("--match", default=None,
                    help="select dispatches whose kernel name contains this text (default: --kernel), e.g. "
                         "one template instance")
    ap.add_argument("--command", required=True)
    ap.add_argument("--out", required=True)
    a = ap.parse_args()
    cf, _ = counter_avg(a.copy_fetch, COPY_KERNEL, "FETCH_SIZE")
    cw, _ = counter_avg(a.copy_write, COPY_KERNEL, "WRITE_SIZE")
    f_scale = COPY_BYTES / (cf * 1024)
    w_scale = COPY_BYTES / (cw * 1024)
    sel = a.match or a.kernel
    kf, nf = counter_avg(a.fetch, sel, "FETCH_SIZE", a.first, a.last)
    kw, nw = counter_avg(a.write, sel, "WRITE_SIZE", a.first, a.last)
    read = kf * 1024 * f_scale
    written = kw * 1024 * w_scale
    rec = {
        "kernel": a.kernel,
        "match": sel,
        "command": a.command,
        "dispatches": {"fetch_pass": nf, "write_pass": nw},
        "fetch_kib_per_dispatch": kf,
        "write_kib_per_dispatch": kw,
        "copy_calibration": {"bytes": COPY_BYTES, "fetch_kib": cf, "write_kib": cw, "fetch_scale": f_scale,
                             "write_scale": w_scale},
        "hbm_read_bytes_per_dispatch": read,
        "hbm_write_bytes_per_dispatch": written,
        "traffic_bytes_per_dispatch": read + written,
        "sources_sha256": sources_sha256(a.kernel),
    }
    if a.algorithmic_bytes:
        rec["algorithmic_bytes_per_dispatch"] = a.algorithmic_bytes
        rec["traffic_over_algorithmic"] = (read + written) / a.algorithmic_bytes
    with open(a.out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
