"""Summaries of rocprofv3 CSV output for this library's kernels.

    python -m block_scaled_precision_mm_amd.profsum kernels DIR
        per-kernel dispatch count and average / min / max duration (us) from
        the *_kernel_stats.csv (or *_kernel_trace.csv) that
        ``rocprofv3 --kernel-trace --stats --output-format csv -d DIR`` writes;

    python -m block_scaled_precision_mm_amd.profsum counters DIR [DIR ...]
        per-kernel average of every counter in the *_counter_collection.csv
        files that ``rocprofv3 --pmc ... --output-format csv -d DIR`` writes;

    python -m block_scaled_precision_mm_amd.profsum vs-aten DIR LOG
        device time per call of ATen's MX product and of this library's, shape
        by shape, from the kernel trace of ``python3 -m
        block_scaled_precision_mm_amd.vs_aten > LOG`` run under ``rocprofv3
        --kernel-trace --output-format csv -d DIR``, and the geometric mean of
        the ratio per format;

    python -m block_scaled_precision_mm_amd.profsum traffic --workload W --kernel-match S \\
            --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR --copy-bytes B
        HBM bytes per launch of the kernel whose name contains S: FETCH_SIZE
        and WRITE_SIZE (KiB per dispatch) each scaled by bytes / counter of a
        plain device copy of B bytes measured the same way; merges the result
        into profiles/traffic.json together with a digest of the HIP sources,
        so that the benchmark only reports it for the kernels it was taken on.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import math
import os
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _rows(pattern_dir, suffix):
    files = sorted(glob.glob(os.path.join(pattern_dir, "**", "*" + suffix), recursive=True))
    for path in files:
        with open(path, newline="") as f:
            yield from csv.DictReader(f)


def _col(row, *names):
    low = {k.lower(): k for k in row}
    for n in names:
        if n.lower() in low:
            return row[low[n.lower()]]
    raise KeyError("none of %s in %s" % (names, list(row)))


def kernels(d):
    out = []
    stats = list(_rows(d, "_kernel_stats.csv"))
    if stats:
        for r in stats:
            out.append((_col(r, "Name", "KernelName"), int(_col(r, "Calls")),
                        float(_col(r, "AverageNs")) / 1e3, float(_col(r, "MinNs")) / 1e3,
                        float(_col(r, "MaxNs")) / 1e3))
    else:
        acc = defaultdict(list)
        for r in _rows(d, "_kernel_trace.csv"):
            t = (int(_col(r, "End_Timestamp")) - int(_col(r, "Start_Timestamp"))) / 1e3
            acc[_col(r, "Kernel_Name")].append(t)
        for name, ts in acc.items():
            out.append((name, len(ts), sum(ts) / len(ts), min(ts), max(ts)))
    return out


def counters(dirs):
    acc = defaultdict(lambda: defaultdict(list))
    for d in dirs:
        for r in _rows(d, "_counter_collection.csv"):
            acc[_col(r, "Kernel_Name")][_col(r, "Counter_Name")].append(float(_col(r, "Counter_Value")))
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in acc.items()}


def _one(cmap, match, counter):
    hits = [(k, v[counter]) for k, v in cmap.items() if match in k and counter in v]
    if len(hits) != 1:
        raise SystemExit("expected one kernel matching %r with %s, found %d" % (match, counter, len(hits)))
    return hits[0][1]


def vs_aten(d, log):
    """Rows (fmt, M, N, K, aten_us, lib_us, aten_kernels_per_call, aten_kernel,
    max_diff_over_max) and the shapes ATen rejected; phases are the kernels
    between two launches of the library's empty kernel, ATen's then the
    library's for each timed shape of the log."""
    recs = [json.loads(l) for l in open(log) if l.startswith("{")]
    timed = [r for r in recs if "calls" in r]
    trace = sorted(_rows(d, "_kernel_trace.csv"), key=lambda r: int(_col(r, "Start_Timestamp")))
    phases, cur, inside = [], [], False
    for r in trace:
        if "mx_empty_kernel" in _col(r, "Kernel_Name"):
            if inside:
                phases.append(cur)
            cur, inside = [], not inside
        elif inside:
            cur.append(r)
    if len(phases) != 2 * len(timed):
        raise SystemExit("expected %d phases, found %d" % (2 * len(timed), len(phases)))
    rows = []
    for k, r in enumerate(timed):
        t = []
        for ph in phases[2 * k: 2 * k + 2]:
            ns = sum(int(_col(x, "End_Timestamp")) - int(_col(x, "Start_Timestamp")) for x in ph)
            t.append(ns / r["calls"] / 1e3)
        names = sorted({_col(x, "Kernel_Name") for x in phases[2 * k]})
        rows.append((r["fmt"], r["M"], r["N"], r["K"], t[0], t[1], len(phases[2 * k]) / r["calls"],
                     names[0] if len(names) == 1 else "%d kernels" % len(names), r["max_diff_over_max"]))
    return rows, [r for r in recs if "aten_error" in r]


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    k = sub.add_parser("kernels")
    k.add_argument("dir")
    c = sub.add_parser("counters")
    c.add_argument("dirs", nargs="+")
    t = sub.add_parser("traffic")
    for a in ("--workload", "--kernel-match", "--fetch", "--write", "--copy-fetch", "--copy-write"):
        t.add_argument(a, required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--copy-match", default="copyBuffer", help="name of the copy kernel")
    t.add_argument("--kernel-name", default=None, help="variant name recorded with the figure")
    t.add_argument("--out", default=os.path.join(ROOT, "profiles", "traffic.json"))
    v = sub.add_parser("vs-aten")
    v.add_argument("dir")
    v.add_argument("log")
    args = ap.parse_args(argv)

    if args.cmd == "vs-aten":
        rows, rejected = vs_aten(args.dir, args.log)
        print("%-4s %5s %6s %6s %10s %10s %7s  %-9s %s" % ("fmt", "M", "N", "K", "aten_us", "lib_us",
                                                            "ratio", "diff/max", "ATen kernel"))
        seen, logs = set(), defaultdict(list)
        for fmt, M, N, K, ta, tl, kpc, kname, diff in rows:
            print("%-4s %5d %6d %6d %10.2f %10.2f %7.2f  %.1e  %s (%.1f per call)" % (
                fmt, M, N, K, ta, tl, ta / tl, diff, kname[:48], kpc))
            if (fmt, M, N, K) not in seen:
                seen.add((fmt, M, N, K))
                logs[fmt].append(math.log(ta / tl))
        for fmt, lv in sorted(logs.items()):
            print("%s: geometric mean of ATen time / library time over %d shapes: %.3f" % (
                fmt, len(lv), math.exp(sum(lv) / len(lv))))
        for r in rejected:
            print("not taken by ATen: %s %dx%dx%d (%s)" % (r["fmt"], r["M"], r["N"], r["K"], r["aten_error"]))
        return

    if args.cmd == "kernels":
        print("%-100s %6s %10s %10s %10s" % ("kernel", "calls", "avg_us", "min_us", "max_us"))
        for name, n, avg, lo, hi in sorted(kernels(args.dir), key=lambda x: -x[1] * x[2]):
            print("%-100s %6d %10.3f %10.3f %10.3f" % (name[:100], n, avg, lo, hi))
    elif args.cmd == "counters":
        for name, cs in counters(args.dirs).items():
            print(name[:100], " ".join("%s=%.6g" % kv for kv in sorted(cs.items())))
    else:
        fetch = _one(counters([args.fetch]), args.kernel_match, "FETCH_SIZE")
        write = _one(counters([args.write]), args.kernel_match, "WRITE_SIZE")
        cf = counters([args.copy_fetch])
        cw = counters([args.copy_write])
        copy_kernels = [k for k in cf if args.copy_match in k]
        if len(copy_kernels) != 1:
            raise SystemExit("expected one copy kernel, found %s" % list(cf))
        ck = copy_kernels[0]
        f_scale = args.copy_bytes / (cf[ck]["FETCH_SIZE"] * 1024.0)
        w_scale = args.copy_bytes / (cw[ck]["WRITE_SIZE"] * 1024.0)
        sys.path.insert(0, ROOT)
        import bench
        rec = {
            "kernel": args.kernel_name,
            "source_digest": bench.kernel_source_digest(args.kernel_name),
            "fetch_kib_per_dispatch": fetch, "write_kib_per_dispatch": write,
            "copy_kernel": ck, "copy_bytes": args.copy_bytes,
            "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
            "hbm_read_bytes_per_launch": int(fetch * 1024 * f_scale),
            "hbm_write_bytes_per_launch": int(write * 1024 * w_scale),
        }
        rec["hbm_bytes_per_launch"] = rec["hbm_read_bytes_per_launch"] + rec["hbm_write_bytes_per_launch"]
        db = {}
        if os.path.exists(args.out):
            with open(args.out) as f:
                db = json.load(f)
        db[args.workload] = rec
        with open(args.out, "w") as f:
            json.dump(db, f, indent=1, sort_keys=True)
            f.write("\n")
        print(json.dumps(rec, indent=1))


if __name__ == "__main__":
    main()
