"""Summarise rocprofv3 CSV output of bench.py into profiles/.

    python -m paged_kv_cache_119_amd.rocprof_summary tables --title T --run LABEL trace|pmc DIR ... \\
        --command "..." --out profiles/X.md [--occupancy KEY LABEL KERNEL]

writes tables of kernel traces and counter passes (and, with --occupancy,
the measured waves per SIMD bench.py reports beside HIP's figure);

    python -m paged_kv_cache_119_amd.rocprof_summary \\
        --trace DIR_WITH_kernel_stats.csv --fetch DIR_WITH_FETCH_counter_collection.csv \\
        --write DIR_WITH_WRITE_counter_collection.csv --config opt13b --partition-size 0 \\
        --algorithmic-bytes N --command "..." [--command "..."] --out profiles/decode_balanced_opt13b.md

Writes a short Markdown summary (mean kernel durations from the kernel trace;
HBM bytes per dispatch from FETCH_SIZE / WRITE_SIZE, each scaled by what the
same counter reads for the 1 GiB device copy bench.py runs with
--copy-calibration) and the traffic record bench.py reports while the decode
kernel sources are unchanged.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_SOURCES = ("paged_kv_cache_119_amd/csrc/decode.hip", "paged_kv_cache_119_amd/csrc/pkv_device.h",
                  "paged_kv_cache_119_amd/csrc/pkv_launch.h", "paged_kv_cache_119_amd/csrc/pkv_split.h")
COPY_BYTES_KIB = (1 << 30) / 1024.0


def kernel_hash(root: str = ROOT) -> str:
    """Hash of the decode kernel sources: a traffic record is valid only for them."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(root, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def library_hash(root: str = ROOT) -> str:
    """Hash of every library source (kernels and C ABI): an occupancy record is
    valid only for them."""
    h = hashlib.sha256()
    for path in sorted(glob.glob(os.path.join(root, "paged_kv_cache_119_amd", "csrc", "*"))):
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


OCCUPANCY_FILE = os.path.join(ROOT, "profiles", "occupancy_counters.json")


def short_name(kernel: str) -> str:
    """`decode_balanced_kernel<0, 128, 16, 4, true, true>` from the demangled name."""
    k = kernel.replace("void ", "").replace("pkv::(anonymous namespace)::", "")
    return k.split("(pkv::DecodeParams")[0]


def occupancy_lines(agg: dict) -> list:
    """Markdown rows of MeanOccupancyPerActiveCU per library kernel."""
    out = ["| kernel | dispatches | waves per SIMD |", "|---|---|---|"]
    for (k, c), v in sorted(agg.items()):
        if c == "MeanOccupancyPerActiveCU" and "pkv" in k:
            out.append(f"| `{short_name(k)}` | {len(v)} | {sum(v) / len(v):.3f} |")
    return out


def record_occupancy(agg: dict, key: str, kernel: str, summary: str) -> None:
    """Store the measured occupancy of `kernel` under `key` for bench.py."""
    hits = [v for (k, c), v in agg.items() if c == "MeanOccupancyPerActiveCU" and kernel in k]
    if not hits:
        raise RuntimeError(f"no MeanOccupancyPerActiveCU for {kernel}")
    rec = {}
    if os.path.exists(OCCUPANCY_FILE):
        with open(OCCUPANCY_FILE) as f:
            rec = json.load(f)
    # The derived counter is SQ_WAVE_CYCLES / SQ_BUSY_CU_CYCLES, both counted
    # per SIMD: on gfx950 it reads in waves per SIMD (a plain streaming read
    # of 131072 waves reads about 7.1 of the 8 slots).
    rec[key] = {"kernel": kernel, "waves_per_simd": round(sum(hits[0]) / len(hits[0]), 3),
                "library_hash": library_hash(),
                "counter": "MeanOccupancyPerActiveCU (SQ_WAVE_CYCLES / SQ_BUSY_CU_CYCLES)",
                "summary": os.path.relpath(summary, ROOT)}
    with open(OCCUPANCY_FILE, "w") as f:
        json.dump(dict(sorted(rec.items())), f, indent=2)


def step_timeline(trace_dir: str, kernel: str) -> list:
    """Markdown lines: median duration of `kernel` and of the launch after it,
    and the median gaps between them, from the dispatch timestamps."""
    import statistics
    hits = sorted(glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True))
    if not hits:
        return []
    rows = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"])
                  for r in csv.DictReader(open(hits[0])))
    split, after, gap_in, gap_out, name = [], [], [], [], None
    for i in range(1, len(rows) - 1):
        a, b, c = rows[i], rows[i + 1], rows[i - 1]
        if kernel in a[2] and "pkv" in a[2] and "pkv" in b[2] and kernel not in b[2]:
            split.append(a[1] - a[0])
            after.append(b[1] - b[0])
            gap_in.append(b[0] - a[1])
            name = short_name(b[2])
            if "pkv" in c[2] and kernel not in c[2]:
                gap_out.append(a[0] - c[1])
    if not split:
        return []
    med = lambda v: statistics.median(v) / 1e3  # noqa: E731
    lines = ["## Step timeline (kernel trace timestamps, medians over the timed steps)", "",
             f"| `{kernel}` | gap | `{name}` | gap to the next step's `{kernel}` | step |", "|---|---|---|---|---|",
             f"| {med(split):.2f} us | {med(gap_in):.2f} us | {med(after):.2f} us | "
             f"{med(gap_out) if gap_out else float('nan'):.2f} us | "
             f"{med(split) + med(gap_in) + med(after) + (med(gap_out) if gap_out else 0.0):.2f} us |", ""]
    return lines


def tables_main(argv) -> int:
    """Markdown tables from several rocprofv3 runs (kernel traces and counter
    passes), optionally with the measured occupancy recorded for bench.py."""
    ap = argparse.ArgumentParser(prog="rocprof_summary tables")
    ap.add_argument("--title", required=True)
    ap.add_argument("--run", action="append", nargs=3, metavar=("LABEL", "KIND", "DIR"), required=True,
                    help="KIND: trace (--kernel-trace --stats) or pmc (--pmc)")
    ap.add_argument("--command", action="append", required=True)
    ap.add_argument("--note", action="append", default=[])
    ap.add_argument("--out", required=True)
    ap.add_argument("--occupancy", action="append", nargs=3, metavar=("KEY", "LABEL", "KERNEL"), default=[],
                    help="record MeanOccupancyPerActiveCU (waves per SIMD) of KERNEL in run LABEL under KEY for bench.py")
    args = ap.parse_args(argv)
    lines = [f"# rocprofv3 summary: {args.title}", "", "Commands (from the repository root, on one MI355X):", ""]
    lines += [f"    {c}" for c in args.command]
    pmc = {}
    for label, kind, d in args.run:
        if kind == "trace":
            lines += ["", f"## {label}: kernel trace", "", "| kernel | calls | mean us | min us | max us |",
                      "|---|---|---|---|---|"]
            for r in kernel_stats(d):
                if "pkv" in r["name"]:
                    lines.append(f"| `{short_name(r['name'])}` | {r['calls']} | {r['avg_us']:.2f} | "
                                 f"{r['min_us']:.2f} | {r['max_us']:.2f} |")
        else:
            agg = counter_means(d)
            pmc[label] = agg
            counters = sorted({c for (_, c) in agg})
            lines += ["", f"## {label}: counters (mean per dispatch)", "",
                      "| kernel | dispatches | " + " | ".join(counters) + " |",
                      "|---|---|" + "---|" * len(counters)]
            for k in sorted({k for (k, _) in agg if "pkv" in k}):
                vals = []
                n = 0
                for c in counters:
                    v = agg.get((k, c), [])
                    n = max(n, len(v))
                    vals.append(f"{sum(v) / len(v):,.3f}" if v else "-")
                lines.append(f"| `{short_name(k)}` | {n} | " + " | ".join(vals) + " |")
    lines += [""] + [f"{n}" for n in args.note] + [""]
    with open(args.out, "w") as f:
        f.write("\n".join(lines))
    for key, label, kernel in args.occupancy:
        record_occupancy(pmc[label], key, kernel, args.out)
    print(args.out)
    return 0


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def kernel_stats(trace_dir: str) -> list:
    rows = list(csv.DictReader(open(_one(os.path.join(trace_dir, "**", "*kernel_stats.csv")))))
    out = []
    for r in rows:
        out.append({"name": r["Name"], "calls": int(r["Calls"]), "avg_us": float(r["AverageNs"]) / 1e3,
                    "min_us": float(r["MinNs"]) / 1e3, "max_us": float(r["MaxNs"]) / 1e3})
    return out


def counter_means(counter_dir: str) -> dict:
    rows = list(csv.DictReader(open(_one(os.path.join(counter_dir, "**", "*counter_collection.csv")))))
    agg = {}
    for r in rows:
        agg.setdefault((r["Kernel_Name"], r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    return agg


def copy_scale(agg: dict, counter: str) -> float:
    """KiB the counter reports for the 1 GiB calibration copy -> scale to true bytes."""
    vals = [max(v) for (k, c), v in agg.items() if c == counter and "copyBuffer" in k]
    if not vals:
        raise RuntimeError(f"no calibration copy found for {counter}")
    return COPY_BYTES_KIB / max(vals)


def main(argv=None) -> int:
    import sys
    argv = sys.argv[1:] if argv is None else argv
    if argv and argv[0] == "tables":
        return tables_main(argv[1:])
    ap = argparse.ArgumentParser()
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", default=None, help="WRITE_SIZE run (omit to report fetched bytes only)")
    ap.add_argument("--config", default="opt13b")
    ap.add_argument("--partition-size", type=int, default=0)
    ap.add_argument("--separate-append", action="store_true")
    ap.add_argument("--kernel", default="decode_balanced_kernel")
    ap.add_argument("--algorithmic-bytes", type=int, required=True)
    ap.add_argument("--command", action="append", required=True,
                    help="a command the profiles were taken with (repeat for each run)")
    ap.add_argument("--out", required=True)
    ap.add_argument("--fetch-scale", type=float, default=None,
                    help="FETCH_SIZE scale measured in another run (when this run has no calibration copy)")
    ap.add_argument("--occ", default=None, help="MeanOccupancyPerActiveCU run of the same command")
    ap.add_argument("--occ-key", default=None, help="record the kernel's occupancy under this key for bench.py")
    ap.add_argument("--note", action="append", default=[])
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic_decode_partition_opt13b.json"),
                    help="record for bench.py's traffic field ('none': write no record)")
    args = ap.parse_args(argv)

    stats = kernel_stats(args.trace)
    fetch = counter_means(args.fetch)
    write = counter_means(args.write) if args.write else {}
    fs = args.fetch_scale if args.fetch_scale is not None else copy_scale(fetch, "FETCH_SIZE")
    ws = copy_scale(write, "WRITE_SIZE") if args.write else None

    def per_dispatch(agg, counter, scale):
        out = {}
        for (k, c), v in agg.items():
            if c == counter and "pkv" in k:
                out[k] = sum(v) / len(v) * scale * 1024.0
        return out

    fb = per_dispatch(fetch, "FETCH_SIZE", fs)
    wb = per_dispatch(write, "WRITE_SIZE", ws) if args.write else {}
    main_k = [k for k in fb if args.kernel in k]
    if not main_k:
        raise RuntimeError(f"kernel {args.kernel} not in the counter output")
    traffic = fb[main_k[0]] + wb.get(main_k[0], 0.0)

    lines = [f"# rocprofv3 summary: {args.kernel}, {args.config} workload", "",
             "Commands (from the repository root, on one MI355X):", ""]
    lines += [f"    {c}" for c in args.command]
    lines += ["",
             "## Kernel trace (rocprofv3 --kernel-trace --stats)", "",
             "| kernel | calls | mean us | min us | max us |", "|---|---|---|---|---|"]
    for r in stats:
        if "pkv" in r["name"]:
            lines.append(f"| `{r['name'][:100]}` | {r['calls']} | {r['avg_us']:.2f} | {r['min_us']:.2f} | "
                         f"{r['max_us']:.2f} |")
    if args.write:
        lines += ["", "## HBM traffic per dispatch (rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE)", "",
                  f"Scale factors from the 1 GiB device copy in the same runs: FETCH_SIZE x {fs:.4f}, "
                  f"WRITE_SIZE x {ws:.4f}.", "",
                  "| kernel | fetched MB | written MB |", "|---|---|---|"]
        for k in sorted(fb):
            lines.append(f"| `{k[:100]}` | {fb[k] / 1e6:.2f} | {wb.get(k, 0.0) / 1e6:.2f} |")
        what = "measured traffic"
    else:
        how = "given" if args.fetch_scale is not None else "from the 1 GiB device copy in the same run"
        lines += ["", "## HBM bytes fetched per dispatch (rocprofv3 --pmc FETCH_SIZE)", "",
                  f"FETCH_SIZE scale x {fs:.4f} ({how}); no WRITE_SIZE run.", "",
                  "| kernel | fetched MB |", "|---|---|"]
        for k in sorted(fb):
            lines.append(f"| `{k[:100]}` | {fb[k] / 1e6:.2f} |")
        what = "measured fetch"
    lines += ["", f"Algorithmic bytes of one `{args.kernel}` launch: {args.algorithmic_bytes / 1e6:.2f} MB; "
              f"{what} {traffic / 1e6:.2f} MB ({traffic / args.algorithmic_bytes:.3f}x).", ""]
    lines += step_timeline(args.trace, args.kernel)
    occ = counter_means(args.occ) if args.occ else None
    if occ is not None:
        lines += ["## Occupancy (rocprofv3 --pmc MeanOccupancyPerActiveCU, mean per dispatch)", ""]
        lines += occupancy_lines(occ) + [""]
    lines += [f"{n}" for n in args.note] + ([""] if args.note else [])
    os.makedirs(os.path.dirname(os.path.abspath(args.out)), exist_ok=True)
    with open(args.out, "w") as f:
        f.write("\n".join(lines))
    if occ is not None and args.occ_key:
        record_occupancy(occ, args.occ_key, args.kernel, args.out)
    if args.traffic_json == "none":
        print(args.out, f"traffic {traffic / 1e6:.2f} MB")
        return 0
    rec = {"kernel": args.kernel, "config": args.config, "partition_size": args.partition_size,
           "separate_append": args.separate_append, "kernel_hash": kernel_hash(),
           "hbm_bytes_per_launch": round(traffic), "fetch_bytes": round(fb[main_k[0]]),
           "write_bytes": round(wb.get(main_k[0], 0.0)), "fetch_scale": fs, "write_scale": ws,
           "commands": args.command}
    with open(args.traffic_json, "w") as f:
        json.dump(rec, f, indent=2)
    print(args.out, args.traffic_json, f"traffic {traffic / 1e6:.2f} MB")
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
