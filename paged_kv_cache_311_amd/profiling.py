"""Summaries of rocprofv3 runs of bench.py, for the profiles/ folder.

Turns the CSV output of
  * `rocprofv3 --kernel-trace --stats ...`  (per-dispatch durations) and
  * `rocprofv3 --pmc FETCH_SIZE ...` / `--pmc WRITE_SIZE ...`
    (HBM bytes per dispatch, in KiB, for the workload and for a plain copy of
    known size that calibrates the counters)
into short markdown summaries and into profiles/decode_traffic.json, the
measured HBM bytes per paged_attention_decode call that bench.py reports as
`roofline.traffic` while the kernel source is unchanged (its sha256 is
recorded beside the numbers).

    python -m paged_kv_cache_311_amd.profiling trace  TRACE_DIR  OUT.md  "CMD"
    python -m paged_kv_cache_311_amd.profiling traffic OUT.json OUT.md \\
        --copy-fetch DIR --copy-write DIR --copy-bytes N \\
        --workload NAME FETCH_DIR WRITE_DIR [--workload ...] --cmd "CMD" ...
"""

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import statistics

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCE = os.path.join(HERE, "csrc", "paged_attention.hip")
DECODE_KERNELS = ("paged_decode_kernel", "paged_decode_merge_kernel")
# the shared-prefix call, reported as a workload of its own ("<name> shared prefix")
SHARED_KERNELS = ("shared_prefix_rows_kernel", "shared_prefix_combine_kernel")


def _csv(directory, suffix):
    hits = sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {directory}")
    with open(hits[0]) as f:
        return list(csv.DictReader(f))


def short_name(name):
    base = name.split("(")[0].replace("void ", "")
    return base.replace("pkv::", "")


def kernel_durations(trace_dir):
    """{(kernel, grid): [duration_us, ...]} for this library's kernels."""
    out = collections.defaultdict(list)
    rows = [r for r in _csv(trace_dir, "kernel_trace.csv") if "pkv::" in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))  # in launch order
    for r in rows:
        grid = r.get("Grid_Size_X") or r.get("Grid_Size")
        key = (short_name(r["Kernel_Name"]), int(grid))
        out[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    return out


def counter_values(pmc_dir, match=None):
    """[(kernel, grid, value_kib)] per dispatch of one counter run."""
    rows = []
    for r in _csv(pmc_dir, "counter_collection.csv"):
        name = r["Kernel_Name"]
        if match is not None and not match(name):
            continue
        rows.append((short_name(name), int(r["Grid_Size"]), float(r["Counter_Value"])))
    return rows


def source_sha256(path=KERNEL_SOURCE):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def cmd_trace(args):
    d = kernel_durations(args.trace_dir)
    lines = [f"# Kernel trace: {args.title}", "", "Command:", "", "```", args.cmd, "```", "",
             f"| kernel | grid (threads) | calls | avg us | avg us, last {args.last} calls | "
             "min us | max us |",
             "|---|---|---|---|---|---|---|"]
    for (k, g), v in sorted(d.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{k}` | {g} | {len(v)} | {statistics.mean(v):.1f} | "
                     f"{statistics.mean(v[-args.last:]):.1f} | {min(v):.1f} | {max(v):.1f} |")
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")


def cmd_traffic(args):
    is_copy = lambda n: "copyBuffer" in n or "copy_kernel" in n
    cf = [v for _, _, v in counter_values(args.copy_fetch, lambda n: is_copy(n))]
    cw = [v for _, _, v in counter_values(args.copy_write, lambda n: is_copy(n))]
    if not cf or not cw:
        raise SystemExit("no copy dispatch found in the calibration runs")
    fetch_scale = args.copy_bytes / (statistics.median(cf) * 1024)
    write_scale = args.copy_bytes / (statistics.median(cw) * 1024)
    result = {
        "kernel_source_sha256": source_sha256(),
        "calibration": {
            "copy_bytes_read": args.copy_bytes, "copy_bytes_written": args.copy_bytes,
            "FETCH_SIZE_KiB": statistics.median(cf), "WRITE_SIZE_KiB": statistics.median(cw),
            "fetch_scale": fetch_scale, "write_scale": write_scale,
        },
        "commands": args.cmd,
        "workloads": {},
    }
    lines = [f"# HBM traffic of paged_attention_decode (PMC counters)", "",
             "Counters: `FETCH_SIZE` and `WRITE_SIZE` (KiB per dispatch), one rocprofv3 run "
             "each.  Scaled by what the same counters read for a plain device copy of "
             f"{args.copy_bytes} bytes (read and written once): fetch x{fetch_scale:.4f}, "
             f"write x{write_scale:.4f}.", "", "Commands:", "", "```"]
    lines += args.cmd + ["```", "",
                         "| workload | kernel | dispatches | FETCH KiB | WRITE KiB | "
                         "HBM read MB | HBM write MB |", "|---|---|---|---|---|---|---|"]
    for name, fdir, wdir in args.workload:
        for label, names in ((name, DECODE_KERNELS), (name + " shared prefix", SHARED_KERNELS)):
            dec = lambda n: any(k in n for k in names)
            f = collections.defaultdict(list)
            w = collections.defaultdict(list)
            for k, _, v in counter_values(fdir, dec):
                f[k].append(v)
            for k, _, v in counter_values(wdir, dec):
                w[k].append(v)
            if not f:
                continue
            # a kernel dispatched once or twice beside the measured steps (a
            # comparison call of the bench) is left out
            most = max(len(v) for v in f.values())
            total = 0.0
            per_kernel = {}
            for k in sorted(kk for kk in f if len(f[kk]) * 2 >= most):
                rd = statistics.median(f[k]) * 1024 * fetch_scale
                wr = statistics.median(w.get(k, [0.0])) * 1024 * write_scale
                per_kernel[k] = {"read_bytes": rd, "write_bytes": wr}
                total += rd + wr
                lines.append(f"| {label} | `{k}` | {len(f[k])} | {statistics.median(f[k]):.0f} | "
                             f"{statistics.median(w.get(k, [0.0])):.0f} | {rd / 1e6:.1f} | "
                             f"{wr / 1e6:.1f} |")
            result["workloads"][label] = {"hbm_bytes_per_call": total, "kernels": per_kernel}
    with open(args.out_json, "w") as fo:
        json.dump(result, fo, indent=1)
    with open(args.out_md, "w") as fo:
        fo.write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("trace_dir")
    t.add_argument("out")
    t.add_argument("cmd")
    t.add_argument("--title", default="bench.py")
    t.add_argument("--last", type=int, default=20,
                   help="also average the last N calls of each kernel (launch order)")
    t.set_defaults(fn=cmd_trace)
    c = sub.add_parser("traffic")
    c.add_argument("out_json")
    c.add_argument("out_md")
    c.add_argument("--copy-fetch", required=True)
    c.add_argument("--copy-write", required=True)
    c.add_argument("--copy-bytes", type=int, required=True)
    c.add_argument("--workload", nargs=3, action="append", required=True,
                   metavar=("NAME", "FETCH_DIR", "WRITE_DIR"))
    c.add_argument("--cmd", action="append", default=[])
    c.set_defaults(fn=cmd_traffic)
    a = ap.parse_args()
    a.fn(a)


if __name__ == "__main__":
    main()
