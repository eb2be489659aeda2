"""Per-kernel summaries of rocprofv3 counter runs.

    python -m block_sparse_attention_abs_amd.traffic bytes FETCH.csv WRITE.csv --copy-bytes N [--rdreq RDREQ.csv]
    python -m block_sparse_attention_abs_amd.traffic counters SQ.csv

`bytes`: FETCH.csv and WRITE.csv are rocprofv3 `--pmc FETCH_SIZE` and `--pmc
WRITE_SIZE` counter_collection files of the same command (bench.py with
--calibrate-copy).  Both counters are read in KiB per dispatch and scaled by
what the same counter reads for the runtime's plain device copy of N bytes
(N read, N written), so the figures are bytes as a copy kernel would count
them.  With --rdreq (a `--pmc TCC_EA0_RDREQ_32B TCC_EA0_RDREQ_64B
TCC_EA0_RDREQ_128B TCC_EA0_RDREQ` file of the same command) the read bytes
are also counted from the L2-to-memory read requests by size, 32, 64 and
128 bytes each, unscaled, with the copy's reading as the check of that sum.

`counters`: the mean of every counter per dispatch, per kernel, plus the
occupancy (mean resident waves per CU over the dispatch as a percentage of
the 32 wave slots of a CU, from SQ_WAVE_CYCLES, which counts in units of four
cycles, and GRBM_GUI_ACTIVE) when both are present.
"""
from __future__ import annotations

import argparse
import csv
import re
from collections import defaultdict

CU_NUM = 256          # compute units of the MI355X
XCD_NUM = 8           # GRBM_GUI_ACTIVE is read once per XCD and summed


def per_dispatch_keyed(path, counter):
    """{(dispatch id, kernel name): value} for one counter (summed over the
    rows a dispatch may be split into)."""
    acc = defaultdict(float)
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                acc[(r["Dispatch_Id"], r["Kernel_Name"])] += float(r["Counter_Value"])
    return acc


def per_dispatch(path, counter):
    """{kernel name: [value per dispatch]} for one counter."""
    out = defaultdict(list)
    for (_, name), v in per_dispatch_keyed(path, counter).items():
        out[name].append(v)
    return out


def counter_names(path):
    with open(path, newline="") as f:
        seen = []
        for r in csv.DictReader(f):
            if r["Counter_Name"] not in seen:
                seen.append(r["Counter_Name"])
    return seen


def short(name):
    m = re.search(r"(\w+)(<[^(]*>)?\(", name)
    return (m.group(1) + (m.group(2) or "")) if m else name[:80]


def mean(v):
    return sum(v) / len(v)


def copy_reading(d, copy_regex):
    """Mean reading of the three largest copy dispatches (the calibration
    copies are the largest copies of the command)."""
    vals = [v for k, vs in d.items() if re.search(copy_regex, k) for v in vs]
    vals = sorted(vals)[-3:]
    return sum(vals) / len(vals) if vals else None


def cmd_bytes(a):
    fetch = per_dispatch(a.fetch_csv, "FETCH_SIZE")
    write = per_dispatch(a.write_csv, "WRITE_SIZE")
    cf, cw = copy_reading(fetch, a.copy_regex), copy_reading(write, a.copy_regex)
    if not cf or not cw:
        raise SystemExit("no copy dispatch found for calibration")
    sf = a.copy_bytes / (cf * 1024.0)
    sw = a.copy_bytes / (cw * 1024.0)
    print(f"copy of {a.copy_bytes} B: FETCH_SIZE {cf:.0f} KiB, WRITE_SIZE {cw:.0f} KiB; "
          f"scale {sf:.4f} (read), {sw:.4f} (write)\n")
    rd = None
    if a.rdreq:
        req = {n: per_dispatch_keyed(a.rdreq, n) for n in
               ("TCC_EA0_RDREQ_32B", "TCC_EA0_RDREQ_64B", "TCC_EA0_RDREQ_128B", "TCC_EA0_RDREQ")}
        per = defaultdict(list)     # kernel -> [(bytes, n32, n64, n128, all) per dispatch]
        for key in req["TCC_EA0_RDREQ_32B"]:
            n32, n64, n128, nall = (req[c].get(key, 0.0) for c in req)
            per[key[1]].append((32 * n32 + 64 * n64 + 128 * n128, n32, n64, n128, nall))
        rd = {k: tuple(mean([d[i] for d in v]) for i in range(5)) for k, v in per.items()}
        cr = sorted(d[0] for k, v in per.items() if re.search(a.copy_regex, k) for d in v)[-3:]
        if cr:
            print(f"copy of {a.copy_bytes} B by read requests (32/64/128 B): {mean(cr):.0f} B "
                  f"({mean(cr) / a.copy_bytes:.4f} of the bytes copied)\n")
    head = "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | read bytes | written bytes | total bytes |"
    rule = "|---|---|---|---|---|---|---|"
    if rd is not None:
        head += " read bytes by requests | requests 32 / 64 / 128 B (all) |"
        rule += "---|---|"
    print(head)
    print(rule)
    for k in sorted(fetch):
        if not re.search(a.kernel_regex, short(k)) or k not in write:
            continue
        f = mean(fetch[k])
        wv = mean(write[k])
        rb, wb = f * 1024.0 * sf, wv * 1024.0 * sw
        row = f"| {short(k)} | {len(fetch[k])} | {f:.0f} | {wv:.0f} | {rb:.0f} | {wb:.0f} | {rb + wb:.0f} |"
        if rd is not None:
            r = rd.get(k)
            row += (f" {r[0]:.0f} | {r[1]:.0f} / {r[2]:.0f} / {r[3]:.0f} ({r[4]:.0f}) |" if r else " | |")
        print(row)


def cmd_counters(a):
    names = counter_names(a.csv)
    data = {n: per_dispatch(a.csv, n) for n in names}
    kernels = sorted({k for d in data.values() for k in d if re.search(a.kernel_regex, short(k))})
    occ = "SQ_WAVE_CYCLES" in names and "GRBM_GUI_ACTIVE" in names
    cols = names + (["occupancy %"] if occ else [])
    print("| kernel | dispatches | " + " | ".join(cols) + " |")
    print("|---|---|" + "---|" * len(cols))
    for k in kernels:
        vals = [mean(data[n][k]) if k in data[n] else float("nan") for n in names]
        row = [f"{v:.0f}" if n != "OccupancyPercent" else f"{v:.1f}" for n, v in zip(names, vals)]
        if occ:
            wc, gui = mean(data["SQ_WAVE_CYCLES"][k]), mean(data["GRBM_GUI_ACTIVE"][k]) / XCD_NUM
            row.append(f"{100.0 * 4.0 * wc / gui / CU_NUM / 32.0:.1f}")
        n_disp = max(len(data[n].get(k, [])) for n in names)
        print(f"| {short(k)} | {n_disp} | " + " | ".join(row) + " |")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    b = sub.add_parser("bytes")
    b.add_argument("fetch_csv")
    b.add_argument("write_csv")
    b.add_argument("--copy-bytes", type=int, required=True)
    b.add_argument("--rdreq", default=None)
    b.add_argument("--copy-regex", default=r"copyBuffer|[Cc]opy")
    b.add_argument("--kernel-regex", default=r"k_")
    c = sub.add_parser("counters")
    c.add_argument("csv")
    c.add_argument("--kernel-regex", default=r"k_")
    a = ap.parse_args()
    cmd_bytes(a) if a.cmd == "bytes" else cmd_counters(a)


if __name__ == "__main__":
    main()
