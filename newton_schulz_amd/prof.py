"""Summaries of rocprofv3 output for libmuon kernels.

    python -m newton_schulz_amd.prof stats  <kernel_stats.csv>
    python -m newton_schulz_amd.prof pmc    <counter_collection.csv>
    python -m newton_schulz_amd.prof traffic --fetch F.csv --write W.csv \
        --copy-fetch CF.csv --copy-write CW.csv --copy-bytes N --kernel SUBSTR

`traffic` turns per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the kernels
whose name contains SUBSTR into bytes per launch, each counter scaled by what
it reads for a plain copy of N bytes (copy bytes / counter bytes).
"""
from __future__ import annotations

import argparse
import collections
import csv
import json
import re
import sys


def source_fingerprint(*paths: str) -> str:
    """First 16 hex digits of the SHA-256 of source files (in the order given)
    with their // comments and blank lines removed: a comment edit keeps a
    counter record valid, any code change invalidates it."""
    import hashlib
    lines = []
    for path in paths:
        for line in open(path, encoding="utf-8"):
            code = re.sub(r"//.*", "", line).rstrip()
            if code:
                lines.append(code)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()[:16]


def short(name: str) -> str:
    name = name.replace("void ", "").replace("(anonymous namespace)::", "")
    return re.sub(r"\(.*", "", name)


def stats(path: str, top: int = 25):
    rows = list(csv.DictReader(open(path)))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    print(f"{'kernel':70s} {'calls':>6s} {'avg_us':>10s} {'total_ms':>10s} {'pct':>6s}")
    for r in rows[:top]:
        print(f"{short(r['Name'])[:70]:70s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.1f} "
              f"{float(r['TotalDurationNs']) / 1e6:10.2f} {float(r['Percentage']):6.2f}")
    print(f"total kernel time {total / 1e6:.2f} ms")


def per_kernel(path: str):
    agg = collections.defaultdict(lambda: collections.defaultdict(float))
    cnt = collections.defaultdict(set)
    for r in csv.DictReader(open(path)):
        k = short(r["Kernel_Name"])
        agg[k][r["Counter_Name"]] += float(r["Counter_Value"])
        cnt[k].add(r["Dispatch_Id"])
    return agg, {k: len(v) for k, v in cnt.items()}


def pmc(path: str):
    agg, n = per_kernel(path)
    for k, c in sorted(agg.items()):
        vals = " ".join(f"{name}={v / n[k]:.4g}" for name, v in sorted(c.items()))
        print(f"{k[:70]:70s} dispatches={n[k]:5d} per-dispatch: {vals}")


def counter_total(path: str, counter: str, match: str):
    agg, n = per_kernel(path)
    tot, disp = 0.0, 0
    for k, c in agg.items():
        if match in k and counter in c:
            tot += c[counter]
            disp += n[k]
    return tot, disp


def traffic(a):
    cf, ncf = counter_total(a.copy_fetch, "FETCH_SIZE", a.copy_kernel)
    cw, ncw = counter_total(a.copy_write, "WRITE_SIZE", a.copy_kernel)
    f, nf = counter_total(a.fetch, "FETCH_SIZE", a.kernel)
    w, nw = counter_total(a.write, "WRITE_SIZE", a.kernel)
    # each copy dispatch moves copy_bytes: scale = bytes / counter bytes per dispatch
    sf = a.copy_bytes / (cf / ncf * 1024.0)
    sw = a.copy_bytes / (cw / ncw * 1024.0)
    res = {
        "kernel": a.label or a.kernel,
        "kernel_match": a.kernel,
        "dispatches": nf,
        "fetch_kib_per_dispatch": f / nf,
        "write_kib_per_dispatch": w / nw,
        "copy_bytes": a.copy_bytes,
        "fetch_scale": sf,
        "write_scale": sw,
        "hbm_bytes_per_launch": f / nf * 1024.0 * sf + w / nw * 1024.0 * sw,
    }
    if a.source:
        res["source"] = a.source
        res["source_code_sha256_16"] = source_fingerprint(*a.source)
    json.dump(res, sys.stdout, indent=1)
    print()


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    p = sub.add_parser("pmc")
    p.add_argument("csv")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-fetch", required=True)
    t.add_argument("--copy-write", required=True)
    t.add_argument("--copy-bytes", type=float, required=True)
    t.add_argument("--copy-kernel", default="copy")
    t.add_argument("--kernel", required=True)
    t.add_argument("--source", nargs="+", default=None,
                   help="kernel source files to fingerprint (the kernel and its local headers)")
    t.add_argument("--label", default=None, help="kernel description stored in the record")
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        stats(a.csv)
    elif a.cmd == "pmc":
        pmc(a.csv)
    else:
        traffic(a)


if __name__ == "__main__":
    main()
