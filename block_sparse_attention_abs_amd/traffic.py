"""HBM traffic per kernel dispatch from two rocprofv3 counter runs.

    python -m block_sparse_attention_abs_amd.traffic FETCH.csv WRITE.csv --copy-bytes N

FETCH.csv and WRITE.csv are rocprofv3 `--pmc FETCH_SIZE` and `--pmc
WRITE_SIZE` counter_collection files of the same command (bench.py with
--calibrate-copy).  Both counters are read in KiB per dispatch.  They are
scaled by what the same counter reads for the runtime's plain device copy of
N bytes (N read, N written), so the figures are bytes as a copy kernel would
count them; prints one markdown row per kernel.
"""
from __future__ import annotations

import argparse
import csv
import re
from collections import defaultdict


def per_dispatch(path, counter):
    """{kernel name: [value per dispatch]} for one counter (summed over the
    rows a dispatch may be split into)."""
    acc = defaultdict(float)
    names = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Dispatch_Id"], r["Kernel_Name"])
            acc[key] += float(r["Counter_Value"])
            names[key] = r["Kernel_Name"]
    out = defaultdict(list)
    for key, v in acc.items():
        out[names[key]].append(v)
    return out


def short(name):
    m = re.search(r"(\w+)(<[^(]*>)?\(", name)
    return (m.group(1) + (m.group(2) or "")) if m else name[:80]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("fetch_csv")
    ap.add_argument("write_csv")
    ap.add_argument("--copy-bytes", type=int, required=True)
    ap.add_argument("--copy-regex", default=r"copyBuffer|[Cc]opy")
    ap.add_argument("--kernel-regex", default=r"k_")
    a = ap.parse_args()
    fetch = per_dispatch(a.fetch_csv, "FETCH_SIZE")
    write = per_dispatch(a.write_csv, "WRITE_SIZE")

    def copy_reading(d):
        vals = [v for k, vs in d.items() if re.search(a.copy_regex, k) for v in vs]
        # the copies of the calibration are the largest copy dispatches
        vals = sorted(vals)[-3:]
        return sum(vals) / len(vals) if vals else None

    cf, cw = copy_reading(fetch), copy_reading(write)
    if not cf or not cw:
        raise SystemExit("no copy dispatch found for calibration")
    sf = a.copy_bytes / (cf * 1024.0)
    sw = a.copy_bytes / (cw * 1024.0)
    print(f"copy of {a.copy_bytes} B: FETCH_SIZE {cf:.0f} KiB, WRITE_SIZE {cw:.0f} KiB; "
          f"scale {sf:.4f} (read), {sw:.4f} (write)\n")
    print("| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | read bytes | written bytes | total bytes |")
    print("|---|---|---|---|---|---|---|")
    for k in sorted(fetch):
        if not re.search(a.kernel_regex, short(k)) or k not in write:
            continue
        f = sum(fetch[k]) / len(fetch[k])
        wv = sum(write[k]) / len(write[k])
        rb, wb = f * 1024.0 * sf, wv * 1024.0 * sw
        print(f"| {short(k)} | {len(fetch[k])} | {f:.0f} | {wv:.0f} | {rb:.0f} | {wb:.0f} | {rb + wb:.0f} |")


if __name__ == "__main__":
    main()
